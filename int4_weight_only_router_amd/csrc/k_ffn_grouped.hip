// k_ffn_grouped.hip -- batched-regime grouped GEMMs on FP16 MFMA (K4a, K4b)
// and the batched shared FP16 expert.
//
// Horizon RunMap "03 / Arquitetura", "04 / Resultados" (Grouped executor:
// compact experts computed in groups) and "08": compact INT4 weights with FP16
// scales are converted inside the kernel, FP16 activations, FP32 accumulation.
// With many tokens per expert the expert FFN is a dense contraction, so it
// runs on the matrix cores: each K-step an INT4 tile of the weights is read
// from HBM (16-byte loads of the device layout), converted in registers to
// fp16 (q * s, one rounding), and written to LDS; the gathered activation rows
// are staged in LDS beside it; four waves multiply 64x64 sub-tiles with
// v_mfma_f32_32x32x16_f16.  The expanded tile lives only in LDS.
//
// Work list: (expert, 128-row tile of that expert's sorted rows) x (128
// output columns).  The grid's y extent is an upper bound on the number of
// row tiles; each workgroup finds its (expert, tile) from the offsets.
//
// Modes
//  GATEUP_W4 : A = x rows gathered through perm (token = perm[p] / k),
//              B = fused gate/up blocks, epilogue SwiGLU -> h[p][I] fp16
//  DOWN_W4   : A = h rows (sorted order), B = down blocks -> y[p][H] fp16
//  GATEUP_F16: shared expert, A = x rows, B = Wg/Wu fp16 row-major -> h fp16
//  DOWN_F16  : shared expert, A = h rows, B = Wd fp16 row-major -> out fp32
#include "moe_common.h"

namespace moe {

enum { GM_GATEUP_W4 = 0, GM_DOWN_W4 = 1, GM_GATEUP_F16 = 2, GM_DOWN_F16 = 3 };

constexpr int BM = 128, BN = 128, BK = 64, KPAD = 8, LDK = BK + KPAD;
constexpr int GEMM_THREADS = 256;
constexpr size_t GEMM_LDS = (size_t)2 * (BM + BN) * LDK * sizeof(_Float16) + BM * sizeof(int);

struct GemmArgs {
    const _Float16 *A;           // activations: x [T][K] or h [rows][K]
    const int32_t *perm;         // GATEUP_W4
    const int32_t *offsets;      // W4 modes: [E+1]
    const uint8_t *const *blobs; // W4 modes
    int64_t off_q, off_s;        // W4: section offsets inside a blob
    const _Float16 *W0, *W1;     // F16 modes: gate/up or down (row-major)
    int k;                       // top-k (token = perm[p] / k)
    int E;                       // experts (1 for the shared expert)
    int rows;                    // total sorted rows (T*k) or tokens (T)
    int K;                       // reduction length
    int NW;                      // W4: 64-row blocks of B per expert matrix (unused for F16)
    int g;                       // group size (W4)
    int ldo;                     // leading dim of the output (I for h, H for y/out)
    void *out;
};

__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int E, int rows,
                                          int target, int lane, int &e_out, int &p0, int &p1)
{
    if (offsets == nullptr) {   // single implicit expert covering all rows
        const int nt = (rows + BM - 1) / BM;
        if (target >= nt)
            return false;
        e_out = 0;
        p0 = target * BM;
        p1 = min(rows, p0 + BM);
        return true;
    }
    int seen = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        int c = 0, o = 0;
        if (e < E) {
            o = offsets[e];
            c = offsets[e + 1] - o;
        }
        const int nt = (c + BM - 1) / BM;
        int incl = nt;
#pragma unroll
        for (int st = 1; st < 64; st <<= 1) {
            int v = __shfl_up(incl, st, 64);
            if (lane >= st)
                incl += v;
        }
        const int total = __shfl(incl, 63, 64);
        if (seen + total > target) {
            const int excl = incl - nt;
            const bool mine = (seen + excl <= target) && (target < seen + incl);
            const uint64_t m = __ballot(mine);
            const int src = __ffsll((long long)m) - 1;
            const int te = __shfl(e, src, 64);
            const int to = __shfl(o, src, 64);
            const int tc = __shfl(c, src, 64);
            const int tx = __shfl(excl, src, 64);
            e_out = te;
            p0 = to + (target - seen - tx) * BM;
            p1 = min(to + tc, p0 + BM);
            return true;
        }
        seen += total;
    }
    return false;
}

template <int MODE>
__global__ __launch_bounds__(GEMM_THREADS) void grouped_gemm_kernel(GemmArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    _Float16 *As = reinterpret_cast<_Float16 *>(smem);                 // [2][BM][LDK]
    _Float16 *Bs = As + 2 * BM * LDK;                                  // [2][BN][LDK]
    int *srow = reinterpret_cast<int *>(Bs + 2 * BN * LDK);            // [BM]
    __shared__ int s_e, s_p0, s_p1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb = blockIdx.x;   // output column tile (128 columns)

    if (wave == 0) {
        int e = -1, p0 = 0, p1 = 0;
        const bool ok = find_tile((MODE == GM_GATEUP_W4 || MODE == GM_DOWN_W4) ? a.offsets
                                                                               : nullptr,
                                  a.E, a.rows, blockIdx.y, lane, e, p0, p1);
        if (lane == 0) {
            s_e = ok ? e : -1;
            s_p0 = p0;
            s_p1 = p1;
        }
    }
    __syncthreads();
    const int e = s_e;
    if (e < 0)
        return;
    const int p0 = s_p0, mrows = s_p1 - s_p0;
    for (int i = tid; i < BM; i += GEMM_THREADS) {
        int src = -1;
        if (i < mrows) {
            const int p = p0 + i;
            src = (MODE == GM_GATEUP_W4) ? a.perm[p] / a.k : p;
        }
        srow[i] = src;
    }
    __syncthreads();

    const int K = a.K;
    const int nk = K / BK;

    // ---- B source for this workgroup
    const uint8_t *blob = nullptr;
    if (MODE == GM_GATEUP_W4 || MODE == GM_DOWN_W4)
        blob = a.blobs[e];

    // A staging: 4 x 16 B per thread; B staging: 1 x 16 B (W4) or 4 x 16 B (F16)
    uint4_t ra[4];
    uint4_t rb[4];
    float rsc = 0.0f;

    auto load_stage = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sgi = tid + GEMM_THREADS * i;   // 0..1023
            const int r = sgi >> 3, ks = sgi & 7;
            const int src = srow[r];
            if (src >= 0)
                ra[i] = *reinterpret_cast<const uint4_t *>(a.A + (size_t)src * K + k0 + ks * 8);
            else
                ra[i] = uint4_t{0u, 0u, 0u, 0u};
        }
        if (MODE == GM_GATEUP_W4 || MODE == GM_DOWN_W4) {
            const int blk = tid >> 7, ch = (tid >> 6) & 1, row = tid & 63;
            const int bidx = nb * 2 + blk;           // 64-row block within the expert matrix
            const int kc = (k0 >> 5) + ch;           // 32-element chunk
            const uint4_t *q = reinterpret_cast<const uint4_t *>(blob + a.off_q);
            rb[0] = q[((size_t)bidx * (K / 32) + kc) * 64 + row];
            const uint16_t *sc = reinterpret_cast<const uint16_t *>(blob + a.off_s);
            rsc = h2f(sc[((size_t)bidx * (K / a.g) + (kc * 32) / a.g) * 64 + row]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sgi = tid + GEMM_THREADS * i;
                const int n = sgi >> 3, ks = sgi & 7;   // GEMM column n of this tile
                const _Float16 *wrow;
                if (MODE == GM_GATEUP_F16) {
                    const int blk = n >> 6, rr = n & 63;
                    const int irow = (nb * 2 + blk) * 32 + (rr & 31);
                    wrow = ((rr < 32) ? a.W0 : a.W1) + (size_t)irow * K;
                } else {
                    wrow = a.W0 + (size_t)(nb * BN + n) * K;
                }
                rb[i] = *reinterpret_cast<const uint4_t *>(wrow + k0 + ks * 8);
            }
        }
    };

    auto store_stage = [&](int buf) {
        _Float16 *as = As + buf * BM * LDK;
        _Float16 *bs = Bs + buf * BN * LDK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sgi = tid + GEMM_THREADS * i;
            const int r = sgi >> 3, ks = sgi & 7;
            *reinterpret_cast<uint4_t *>(as + r * LDK + ks * 8) = ra[i];
        }
        if (MODE == GM_GATEUP_W4 || MODE == GM_DOWN_W4) {
            const int blk = tid >> 7, ch = (tid >> 6) & 1, row = tid & 63;
            const half2_t s2 = {(_Float16)rsc, (_Float16)rsc};
            half2_t q[16];
            nib8_to_h2x4(rb[0].x, q + 0);
            nib8_to_h2x4(rb[0].y, q + 4);
            nib8_to_h2x4(rb[0].z, q + 8);
            nib8_to_h2x4(rb[0].w, q + 12);
#pragma unroll
            for (int m = 0; m < 16; ++m)
                q[m] = q[m] * s2;
            uint4_t *dst = reinterpret_cast<uint4_t *>(bs + (blk * 64 + row) * LDK + ch * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint4_t v;
                v.x = __builtin_bit_cast(uint32_t, q[4 * j + 0]);
                v.y = __builtin_bit_cast(uint32_t, q[4 * j + 1]);
                v.z = __builtin_bit_cast(uint32_t, q[4 * j + 2]);
                v.w = __builtin_bit_cast(uint32_t, q[4 * j + 3]);
                dst[j] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sgi = tid + GEMM_THREADS * i;
                const int n = sgi >> 3, ks = sgi & 7;
                *reinterpret_cast<uint4_t *>(bs + n * LDK + ks * 8) = rb[i];
            }
        }
    };

    const int wm = wave & 1, wn = wave >> 1;
    float16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            load_stage(kt + 1);
        const _Float16 *as = As + cur * BM * LDK;
        const _Float16 *bs = Bs + cur * BN * LDK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kof = kk * 16 + (lane >> 5) * 8;
            half8_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const half8_t *>(
                    as + (wm * 64 + i * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const half8_t *>(
                    bs + (wn * 64 + j * 32 + (lane & 31)) * LDK + kof);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j],
                                                                      0, 0, 0);
        }
        if (kt + 1 < nk)
            store_stage(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  32x32 accumulator layout: value r of lane l is
    // row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
    const int col = lane & 31;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m >= mrows)
                continue;
            const size_t p = (size_t)(p0 + m);
            if (MODE == GM_GATEUP_W4 || MODE == GM_GATEUP_F16) {
                const float gv = acc[i][0][r], uv = acc[i][1][r];
                const float hv = gv / (1.0f + expf(-gv)) * uv;
                const int icol = (nb * 2 + wn) * 32 + col;
                static_cast<_Float16 *>(a.out)[p * a.ldo + icol] = (_Float16)hv;
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int ocol = nb * BN + wn * 64 + j * 32 + col;
                    if (MODE == GM_DOWN_W4)
                        static_cast<_Float16 *>(a.out)[p * a.ldo + ocol] = (_Float16)acc[i][j][r];
                    else
                        static_cast<float *>(a.out)[p * a.ldo + ocol] = acc[i][j][r];
                }
            }
        }
    }
}

template <int MODE>
static int launch_mode(dim3 grid, hipStream_t s, const GemmArgs &a)
{
    static bool attr_set = false;   // raising the LDS limit is idempotent
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void *)grouped_gemm_kernel<MODE>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)GEMM_LDS);
        if (err != hipSuccess)
            return set_error(MOE_EHIP, "hipFuncSetAttribute: %s", hipGetErrorString(err));
        attr_set = true;
    }
    hipLaunchKernelGGL(grouped_gemm_kernel<MODE>, grid, dim3(GEMM_THREADS), GEMM_LDS, s, a);
    MOE_LAUNCH_CHECK("grouped_gemm_kernel");
    return MOE_OK;
}

static unsigned tile_bound(int rows, int E)
{
    const int64_t nt = ((int64_t)rows + BM - 1) / BM + (E > 1 ? std::min<int64_t>(E, rows) : 0);
    return (unsigned)std::max<int64_t>(nt, 1);
}

size_t ffn_batched_ws_bytes(int T, int I, int k)
{
    return (size_t)al256((int64_t)T * k * I * sizeof(_Float16));
}

int launch_ffn_batched(const void *x, const int32_t *perm, const int32_t *offsets,
                       const void *const *blobs, int T, int H, int I, int E, int k, int g,
                       void *y, void *ws, hipStream_t s)
{
    const int rows = T * k;
    if (rows == 0)
        return MOE_OK;
    const DevLayout L = dev_layout(H, I, g);
    _Float16 *h = static_cast<_Float16 *>(ws);
    GemmArgs a{};
    a.perm = perm;
    a.offsets = offsets;
    a.blobs = reinterpret_cast<const uint8_t *const *>(blobs);
    a.k = k;
    a.E = E;
    a.rows = rows;
    a.g = g;
    // gate/up: GEMM N = 2I (fused blocks), K = H, out h [rows][I]
    a.A = static_cast<const _Float16 *>(x);
    a.off_q = L.gu_q;
    a.off_s = L.gu_s;
    a.K = H;
    a.ldo = I;
    a.out = h;
    int rc = launch_mode<GM_GATEUP_W4>(dim3(I / 64, tile_bound(rows, E)), s, a);
    if (rc)
        return rc;
    // down: GEMM N = H, K = I, out y [rows][H] fp16
    a.A = h;
    a.off_q = L.d_q;
    a.off_s = L.d_s;
    a.K = I;
    a.ldo = H;
    a.out = y;
    return launch_mode<GM_DOWN_W4>(dim3(H / 128, tile_bound(rows, E)), s, a);
}

int launch_shared_batched(const void *x, const void *wg, const void *wu, const void *wd, int T,
                          int H, int Is, float *out, void *ws, hipStream_t s)
{
    if (T == 0)
        return MOE_OK;
    _Float16 *h = static_cast<_Float16 *>(ws);
    GemmArgs a{};
    a.E = 1;
    a.rows = T;
    a.A = static_cast<const _Float16 *>(x);
    a.W0 = static_cast<const _Float16 *>(wg);
    a.W1 = static_cast<const _Float16 *>(wu);
    a.K = H;
    a.ldo = Is;
    a.out = h;
    int rc = launch_mode<GM_GATEUP_F16>(dim3(Is / 64, tile_bound(T, 1)), s, a);
    if (rc)
        return rc;
    a.A = h;
    a.W0 = static_cast<const _Float16 *>(wd);
    a.W1 = nullptr;
    a.K = Is;
    a.ldo = H;
    a.out = out;
    return launch_mode<GM_DOWN_F16>(dim3(H / 128, tile_bound(T, 1)), s, a);
}

}  // namespace moe
