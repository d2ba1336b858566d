// k_ffn_small.hip -- small-batch routed expert FFN (2 to 32 tokens) from
// INT4 weights on the matrix cores.
//
// Horizon RunMap "03 / Arquitetura" and "08 / Comportamento do modelo": INT4
// weights with FP16 scales converted inside the kernel, FP16 activations,
// FP32 accumulation, SwiGLU.  "10 / Próximas perguntas" lists simultaneous
// use as an open question; this is the kernel for a handful of concurrent
// token streams.
//
// With T <= 32 tokens an expert holds at most T rows (a token picks an expert
// at most once), so its rows fit one 32-wide MFMA operand, and the cost is
// the expert's weight bytes.  The decode GEMV handles rows one after another
// on the vector ALUs; the tiled grouped GEMM sizes its tiles for hundreds of
// rows.  Here:
//  * a workgroup (four waves) takes one active expert and a group of its
//    64-row weight blocks; the expert's rows (gathered x rows, or its h
//    rows) are staged in LDS, in parts along K when all of them would not
//    leave room for four workgroups per CU;
//  * each wave streams one block's INT4 words from memory into registers,
//    SB_D chunks of 32 K ahead.  In the device layout a lane's 8-byte slice
//    of a chunk row is its B operand for two consecutive 16-K steps, so the
//    words go straight from the load into the fp16(q*s) conversion and then
//    into v_mfma_f32_32x32x16_f16 (weights as the 32-row operand, rows of
//    the expert as the 32-column one, padded by repeating the last row);
//  * when few experts are active the K extent of a block is split over KS
//    waves (sized for about two workgroups per CU from the expected number
//    of active experts) and their fp32 partials are added in LDS in a fixed
//    order;
//  * epilogue as in the grouped GEMM: SwiGLU -> h [rows][I] (gate/up), or
//    y [rows][H] (down), fp16.  h and y are the batched regime's buffers, so
//    the combine step is shared with it.
#include "k_w4_frag.h"

#include <algorithm>
#include <cmath>

namespace moe {

enum { SB_GATEUP = 0, SB_DOWN = 1 };

constexpr int SB_WAVES = 4;   // waves per workgroup
constexpr int SB_WANT = 2;     // K split sized for this many workgroups per CU
constexpr int SB_T = SB_WAVES * 64;
constexpr int SB_D = 8;          // 32-K chunks in flight per wave
constexpr int SB_MAXR = 32;      // rows of one expert (one MFMA column operand)
constexpr int SB_XB = 4;         // 16-byte activation pieces per thread per staging round
constexpr size_t SB_LDS_MAX = 156 * 1024;   // dynamic LDS of one workgroup (static part aside)
constexpr size_t SB_XBUDGET = 40 * 1024;   // staged rows per workgroup: four share a CU

struct SmallArgs {
    const _Float16 *A;             // x [T][K] (gate/up) or h [T*k][K] (down)
    const int32_t *perm;           // gate/up: token of sorted row p is perm[p] / k
    const int32_t *offsets;        // [E+1] sorted-row ranges per expert
    const uint8_t *const *blobs;   // [E] device blobs (null: expert not computed)
    int64_t off_q, off_s;          // weight / scale sections inside a blob
    int64_t off_z;                 // zero points (zero-point format; scales' order, u8)
    int k, E, K, nblk, g, ldo, rmax;
    int phases;                    // the rows are staged in this many parts of K
    _Float16 *out;                 // h [T*k][I] or y [T*k][H]
};

template <int KS>
constexpr int sb_red_floats_per_row()
{
    return (SB_WAVES - SB_WAVES / KS) * 2 * 16 * 2;   // writer waves x 2 tiles x 16 values x 2 halves
}

// LDS: one part of the staged rows, later reused for the K-split partials.
template <int KS>
static size_t sb_lds_bytes(int rmax, int K, int P)
{
    const size_t xs = (size_t)rmax * (K / P + 8) * sizeof(_Float16);
    const size_t red = KS > 1 ? (size_t)rmax * sb_red_floats_per_row<KS>() * sizeof(float) : 0;
    return std::max(xs, red);
}

// Workgroups per CU the register budget is sized for: four (128 VGPRs) for
// symmetric blobs; three (170) with zero points, whose per-chunk offsets
// spilled about 50 registers at four (T = 8: 72 -> 46 us, T = 32: 100 -> 71
// us for the 64-expert layer; the symmetric kernel measures the same or
// slower at three).
constexpr int sb_occupancy(bool zp) { return zp ? 3 : 16 / SB_WAVES; }

template <int MODE, int KS, bool ZP>
__global__ __launch_bounds__(SB_T, sb_occupancy(ZP)) void w4_small_kernel(SmallArgs a)
{
    constexpr bool GATEUP = MODE == SB_GATEUP;
    constexpr int BPW = SB_WAVES / KS;   // weight blocks per workgroup
    static_assert(SB_WAVES % KS == 0, "K split must divide the wave count");

    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_e, s_p0, s_p1;
    __shared__ const uint8_t *s_blob;
    __shared__ int s_src[SB_MAXR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;

    // ---- the blockIdx.y-th expert with rows (ascending ids): wave 0 reads
    // the offsets and blob pointers in one sweep, 16 experts per lane
    // (E <= 1024)
    if (wave == 0) {
        const int e0 = 16 * lane;
        int o[17];
        const uint8_t *bp[16];
#pragma unroll
        for (int j = 0; j <= 16; ++j)
            o[j] = (e0 + j <= a.E) ? ldg(a.offsets + e0 + j) : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            bp[j] = (e0 + j < a.E) ? ldg(a.blobs + e0 + j) : nullptr;
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (e0 + j < a.E && o[j + 1] > o[j])
                m |= 1u << j;
        const int cnt = __popc(m);
        int incl = cnt;
#pragma unroll
        for (int st = 1; st < 64; st <<= 1) {
            const int v = __shfl_up(incl, st, 64);
            if (lane >= st)
                incl += v;
        }
        const int total = __shfl(incl, 63, 64);   // every lane takes part in the shuffle
        const int target = blockIdx.y;
        const int excl = incl - cnt;
        if (target >= excl && target < incl) {
            uint32_t mm = m;
            for (int r = target - excl; r > 0; --r)
                mm &= mm - 1u;
            const int j = __ffs(mm) - 1;
            int p0 = 0, p1 = 0;
            const uint8_t *b = nullptr;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                if (jj == j) {
                    p0 = o[jj];
                    p1 = o[jj + 1];
                    b = bp[jj];
                }
            s_e = e0 + j;
            s_p0 = p0;
            s_p1 = p1;
            s_blob = b;
        }
        if (lane == 0 && target >= total)
            s_e = -1;
    }
    __syncthreads();
    if (s_e < 0 || s_blob == nullptr)
        return;   // fewer active experts than rows of the grid, or not in the table
    const int p0 = s_p0;
    const int R = min(s_p1 - p0, a.rmax);
    const int K = a.K;
    const int P = a.phases;          // the rows are staged P times, K/P columns each
    const int KP = K / P;
    const int LDX = KP + 8;          // LDS row stride in halfs (+16 bytes spreads rows over banks)
    const int gshift = __builtin_ctz((unsigned)a.g);
    const int NKc = K / 32;

    // ---- this wave's weight block and K range.  Wave ks takes the ks-th
    // share of every part: nckp chunks per part.  A wave past the last block
    // streams block 0 and stores nothing, so every wave meets the same
    // barriers.
    const int bw = wave / KS, ks = wave % KS;
    const int blk = (int)blockIdx.x * BPW + bw;
    const bool live = blk < a.nblk;
    const int nckp = NKc / (P * KS);
    const uint64_t ub = reinterpret_cast<uint64_t>(s_blob);
    const uint8_t *blob = reinterpret_cast<const uint8_t *>(
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ub >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ub));
    const int bb = live ? blk : 0;
    const uint8_t *qb = blob + a.off_q + (size_t)bb * NKc * 1024 + col * 16 + half * 8;
    const uint8_t *sb = blob + a.off_s + (size_t)bb * (K >> gshift) * 128 + col * 2;

    const uint8_t *zb = blob + a.off_z + (size_t)bb * (K >> gshift) * 64 + col;

    uint2_t wq[SB_D][2];    // [ring][tile]: rows col and 32 + col of the chunk
    uint16_t sc[SB_D][2];   // their group scales
    uint8_t zc[ZP ? SB_D : 1][2];   // ZP: their zero points
    auto load = [&](int i, int c) {   // c: absolute chunk of the block
        const uint8_t *q = qb + (size_t)c * 1024;
        // expert weights are streamed once per call: non-temporal
        wq[i][0] = ldg_nt(reinterpret_cast<const uint2_t *>(q));
        wq[i][1] = ldg_nt(reinterpret_cast<const uint2_t *>(q + 512));
        const uint8_t *sp = sb + (size_t)((c * 32) >> gshift) * 128;
        sc[i][0] = ldg_nt(reinterpret_cast<const uint16_t *>(sp));
        sc[i][1] = ldg_nt(reinterpret_cast<const uint16_t *>(sp + 64));
        if constexpr (ZP) {
            const uint8_t *zp = zb + (size_t)((c * 32) >> gshift) * 64;
            zc[i][0] = ldg_nt(zp);
            zc[i][1] = ldg_nt(zp + 32);
        }
    };
    // absolute chunk of this wave's f-th chunk in phase ph
    auto chunk_of = [&](int ph, int f) { return ph * (NKc / P) + ks * nckp + f; };
    // Every load of the ring is unconditional (past the end of a part it
    // re-reads the part's last chunk), so the compiler's in-order wait counts
    // stay exact and a chunk's use waits only for its own load.
    auto prologue = [&](int ph) {
#pragma unroll
        for (int i = 0; i < SB_D; ++i)
            load(i, chunk_of(ph, min(i, nckp - 1)));
    };
    prologue(0);

    // ---- the expert's rows, K columns [ph*KP, (ph+1)*KP), into LDS
    if (tid < R)
        s_src[tid] = GATEUP ? ldg(a.perm + p0 + tid) / a.k : p0 + tid;
    __syncthreads();
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    auto stage = [&](int ph) {
        const int per_row = KP / 8;
        const int n = R * per_row;
        for (int i0 = tid; i0 < n; i0 += SB_XB * SB_T) {
            half8_t v[SB_XB];
#pragma unroll
            for (int u = 0; u < SB_XB; ++u) {
                const int i = i0 + u * SB_T;
                if (i < n) {
                    const int r = i / per_row, c = i - r * per_row;
                    v[u] = ldg(reinterpret_cast<const half8_t *>(a.A + (size_t)s_src[r] * K +
                                                                 ph * KP + c * 8));
                }
            }
#pragma unroll
            for (int u = 0; u < SB_XB; ++u) {
                const int i = i0 + u * SB_T;
                if (i < n) {
                    const int r = i / per_row, c = i - r * per_row;
                    *reinterpret_cast<half8_t *>(xs + r * LDX + c * 8) = v[u];
                }
            }
        }
    };

    // ---- stream the block, part by part: stage the rows' part, run the
    // ring over this wave's chunks of it, then request the next part's first
    // chunks before its rows are staged
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
    float16_t acc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[n][r] = 0.0f;
    const _Float16 *xa = xs + min(col, R - 1) * LDX + ks * nckp * 32 + half * 8;
    auto compute = [&](int i, int f) {   // f: chunk within this wave's share of the part
        const f16 s0 = __builtin_bit_cast(f16, sc[i][0]);
        const f16 s1 = __builtin_bit_cast(f16, sc[i][1]);
        half2_t klo0, khi0, klo1, khi1;
        if constexpr (ZP) {
            zp_offsets(zc[i][0], klo0, khi0);
            zp_offsets(zc[i][1], klo1, khi1);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const half8_t av = *reinterpret_cast<const half8_t *>(xa + f * 32 + kh * 16);
            half8_t b0, b1;
            if constexpr (ZP) {
                b0 = dequant8_zp(kh ? wq[i][0].y : wq[i][0].x, half2_t{s0, s0}, magic, klo0, khi0);
                b1 = dequant8_zp(kh ? wq[i][1].y : wq[i][1].x, half2_t{s1, s1}, magic, klo1, khi1);
            } else {
                b0 = dequant8(kh ? wq[i][0].y : wq[i][0].x, half2_t{s0, s0}, magic);
                b1 = dequant8(kh ? wq[i][1].y : wq[i][1].x, half2_t{s1, s1}, magic);
            }
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, av, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, av, acc[1], 0, 0, 0);
        }
    };
    for (int ph = 0; ph < P; ++ph) {
        if (ph > 0) {
            __syncthreads();   // every wave is done with the previous part
            prologue(ph);
        }
        stage(ph);
        __syncthreads();
        int f = 0;
        for (; f + SB_D < nckp; f += SB_D) {
#pragma unroll
            for (int i = 0; i < SB_D; ++i) {
                compute(i, f + i);
                load(i, chunk_of(ph, min(f + SB_D + i, nckp - 1)));
            }
        }
#pragma unroll
        for (int i = 0; i < SB_D; ++i)
            if (f + i < nckp)
                compute(i, f + i);
    }

    // ---- K split: waves ks > 0 hand their partials to wave ks = 0 of the
    // same block, which adds them in ks order
    if constexpr (KS > 1) {
        __syncthreads();   // every wave is done with the staged rows
        float *red = reinterpret_cast<float *>(smem);
        const int rp = a.rmax;
        auto slot = [&](int b, int kk, int n, int r) {
            // [writer][tile][value][half][row]; rows >= R are never touched
            return (((((b * (KS - 1) + kk - 1) * 2 + n) * 16 + r) * 2 + half) * rp) + col;
        };
        if (live && ks > 0 && col < R) {
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    red[slot(bw, ks, n, r)] = acc[n][r];
        }
        __syncthreads();
        if (live && ks == 0 && col < R) {
            for (int kk = 1; kk < KS; ++kk)
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[n][r] += red[slot(bw, kk, n, r)];
        }
    }

    // ---- epilogue: value r of lane l is weight row 8*(r/4) + 4*(l/32) + (r%4)
    // of tile n and expert row l%32, so r = 4j..4j+3 are 4 consecutive
    // output columns (one 8-byte store)
    if (!live || ks != 0 || col >= R)
        return;
    const size_t p = (size_t)(p0 + col);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int cc = 8 * j + 4 * half;
        half4_t v;
        if constexpr (GATEUP) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = (_Float16)swiglu_fast(acc[0][4 * j + i], acc[1][4 * j + i]);
            *reinterpret_cast<half4_t *>(a.out + p * a.ldo + blk * 32 + cc) = v;
        } else {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (_Float16)acc[f][4 * j + i];
                *reinterpret_cast<half4_t *>(a.out + p * a.ldo + blk * 64 + f * 32 + cc) = v;
            }
        }
    }
}

static int sb_num_cus()
{
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

template <int MODE, int KS, bool ZP>
static int launch_small_ks(hipStream_t s, const SmallArgs &a, int active_max)
{
    const size_t lds = sb_lds_bytes<KS>(a.rmax, a.K, a.phases);
    if (lds > SB_LDS_MAX)
        return set_error(MOE_EUNSUPPORTED, "small-batch kernel: %zu bytes of LDS", lds);
    static size_t attr = 0;   // dynamic LDS limit raised so far (idempotent, only grows)
    if (lds > attr) {
        hipError_t err = hipFuncSetAttribute((const void *)w4_small_kernel<MODE, KS, ZP>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess)
            return set_error(MOE_EHIP, "hipFuncSetAttribute: %s", hipGetErrorString(err));
        attr = lds;
    }
    constexpr int BPW = SB_WAVES / KS;
    dim3 grid((unsigned)((a.nblk + BPW - 1) / BPW), (unsigned)active_max);
    hipLaunchKernelGGL((w4_small_kernel<MODE, KS, ZP>), grid, dim3(SB_T), lds, s, a);
    MOE_LAUNCH_CHECK("w4_small_kernel");
    return MOE_OK;
}

// K split: the smallest that gives the grid SB_WANT workgroups per CU for
// the expected number of active experts (uniform routing), keeping at least
// two chunks per wave.
static int pick_ks(double active, int nblk, int nck)
{
    const double want = (double)SB_WANT * sb_num_cus();
    int best = 1;
    for (int ks = 1; ks <= SB_WAVES; ks *= 2) {
        if (nck % ks || nck / ks < 2)
            break;
        best = ks;
        const int bpw = SB_WAVES / ks;
        if (active * ((nblk + bpw - 1) / bpw) >= want)
            break;
    }
    return best;
}

// Parts the staged rows are split into along K: the fewest that keep them
// within SB_XBUDGET (so that several workgroups share a CU), given that a
// wave's chunks of one part must be a multiple of the ring depth.
static int pick_phases(int rmax, int K, int ks)
{
    const int nck = K / 32;
    int best = 1;
    for (int P = 1; P <= 8; P *= 2) {
        if (nck % (P * ks) || (P > 1 && (nck / (P * ks)) % SB_D))
            break;
        best = P;
        if ((size_t)rmax * (K / P + 8) * sizeof(_Float16) <= SB_XBUDGET)
            break;
    }
    return best;
}

template <int MODE, int KS, bool ZP>
static int launch_small_at_most(hipStream_t s, const SmallArgs &a, int active_max, int ks)
{
    if constexpr (KS > 1) {
        if (ks < KS)
            return launch_small_at_most<MODE, KS / 2, ZP>(s, a, active_max, ks);
    }
    return launch_small_ks<MODE, KS, ZP>(s, a, active_max);
}

template <int MODE>
static int launch_small(hipStream_t s, SmallArgs a, int active_max, double active, bool zp)
{
    const int ks = pick_ks(active, a.nblk, a.K / 32);
    a.phases = pick_phases(a.rmax, a.K, ks);
    return zp ? launch_small_at_most<MODE, SB_WAVES, true>(s, a, active_max, ks)
              : launch_small_at_most<MODE, SB_WAVES, false>(s, a, active_max, ks);
}

// The staged rows always fit once split along K (32 rows of at most 8192/8
// halfs), so the regime is open to every supported shape up to 32 tokens.
bool ffn_small_fits(int T, int H, int I)
{
    (void)H;
    (void)I;
    return T >= 0 && T <= SB_MAXR;
}

// Gate/up then down for T <= 32 tokens; h lives in ws (the batched regime's
// workspace), y is [T*k][H] fp16.
int launch_ffn_small(const void *x, const int32_t *perm, const int32_t *offsets,
                     const void *const *blobs, int T, int H, int I, int E, int k, int g, int fmt,
                     void *y, void *ws, hipStream_t s)
{
    const int rows = T * k;
    if (rows == 0)
        return MOE_OK;
    if (!ffn_small_fits(T, H, I))
        return set_error(MOE_EUNSUPPORTED, "small-batch kernel: T=%d with H=%d, I=%d", T, H, I);
    const DevLayout L = dev_layout(H, I, g, fmt);
    const bool zp = fmt == FMT_ZP;
    const int active_max = std::min(E, rows);
    const double active = E * (1.0 - std::pow(1.0 - (double)k / E, (double)T));
    SmallArgs a{};
    a.perm = perm;
    a.offsets = offsets;
    a.blobs = reinterpret_cast<const uint8_t *const *>(blobs);
    a.k = k;
    a.E = E;
    a.g = g;
    a.rmax = T;
    // gate/up: fused 64-row blocks, K = H, out h [rows][I]
    a.A = static_cast<const _Float16 *>(x);
    a.off_q = L.gu_q;
    a.off_s = L.gu_s;
    a.off_z = L.gu_z;
    a.K = H;
    a.nblk = I / 32;
    a.ldo = I;
    a.out = static_cast<_Float16 *>(ws);
    int rc = launch_small<SB_GATEUP>(s, a, active_max, active, zp);
    if (rc)
        return rc;
    // down: H/64 blocks, K = I, out y [rows][H]
    a.A = static_cast<const _Float16 *>(ws);
    a.off_q = L.d_q;
    a.off_s = L.d_s;
    a.off_z = L.d_z;
    a.K = I;
    a.nblk = H / 64;
    a.ldo = H;
    a.out = static_cast<_Float16 *>(y);
    return launch_small<SB_DOWN>(s, a, active_max, active, zp);
}

}  // namespace moe
