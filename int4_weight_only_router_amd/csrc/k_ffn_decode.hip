// k_ffn_decode.hip -- decode-regime routed expert FFN straight from INT4
// weights (K3).
//
// Horizon RunMap "03 / Arquitetura" and "08 / Comportamento do modelo": the
// expert kernel reads compact INT4 weights and FP16 scales, converts the
// values it needs during the computation (here: in registers), multiplies
// with FP16 activations and accumulates in FP32; no expanded copy of an
// expert ever exists.  SwiGLU h = silu(Wg x) * (Wu x), y = Wd h.
//
// Decode kernel layout.  One workgroup per (intermediate slice of 32, active
// expert).  In the device layout a slice is one fused 64-row block (32 gate
// rows + the 32 up rows of the same intermediate indices) whose 32-element
// input chunks are 1 KB contiguous runs: a wave reads one run with one 16-byte
// load per lane, lane = weight row, and every lane dots its 32 nibbles with
// the same 32 activations (broadcast from LDS).  No cross-lane reduction is
// needed along K.  The waves split K, their partial sums meet in LDS, SwiGLU
// is applied, and the 32 fp16 h values then multiply the slice's 32-column
// strip of the down projection (one 1 KB run per 64 output rows).  Each
// workgroup writes an fp32 partial y for its slice; moe_combine adds the
// slices in order.  All weight loads of a workgroup are issued before any
// arithmetic, so a workgroup keeps its whole ~96 KB in flight.
#include "k_decode_frag.h"

namespace moe {

// Finds the a-th expert (in id order) with at least one routed row; -1 if
// none.  The blob pointers are fetched in the same sweep as the offsets, so
// the expert's weight address is known one memory round trip after entry.
__device__ __forceinline__ int nth_active_expert(const int32_t *__restrict__ offsets,
                                                 const uint8_t *const *__restrict__ blobs, int E,
                                                 int a, int lane, const uint8_t **blob_out)
{
    int seen = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const bool inb = e < E;
        const int o0 = inb ? offsets[e] : 0;
        const int o1 = inb ? offsets[e + 1] : 0;
        const uint8_t *bp = inb ? blobs[e] : nullptr;
        const bool act = o1 > o0;
        const uint64_t m = __ballot(act);
        const int n = __popcll(m);
        if (seen + n > a) {
            const int r = a - seen;
            const int rank = __popcll(m & ((1ull << lane) - 1ull));
            const uint64_t hit = __ballot(act && rank == r);
            const int src = __ffsll((long long)hit) - 1;
            *blob_out = reinterpret_cast<const uint8_t *>(
                __shfl(reinterpret_cast<long long>(bp), src, 64));
            return e0 + src;
        }
        seen += n;
    }
    return -1;
}

constexpr int DECODE_XPRE = 4;   // up to this many tokens, all x rows are staged at entry

template <int H, int NW>
__global__ __launch_bounds__(NW * 64) void ffn_decode_kernel(
    const f16 *__restrict__ x, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const uint8_t *const *__restrict__ blobs,
    const uint8_t *const *__restrict__ skip, int I, int E, int k, int g, int ntk,
    int64_t off_guq, int64_t off_dq, int64_t off_gus, int64_t off_ds, float *__restrict__ y)
{
    constexpr int NK = H / 32;                 // input chunks of gate/up rows
    constexpr int CPW = NK / NW;               // chunks per wave
    constexpr int NRB = H / 64;                // 64-row blocks of the down projection
    constexpr int RBW = (NRB + NW - 1) / NW;   // down blocks per wave
    static_assert(NK % NW == 0, "H/32 must be a multiple of the wave count");

    __shared__ __align__(16) half2_t xp[DECODE_XPRE][H / 2];   // prepared activations
    __shared__ float xc[DECODE_XPRE][NK];                     // their chunk constants
    __shared__ float red[NW * 64];
    __shared__ __align__(16) half2_t hp[16];                  // prepared h chunk
    __shared__ float hcorr;
    __shared__ int s_e;
    __shared__ const uint8_t *s_blob;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slice = blockIdx.x;
    const int T = ntk / k;
    const bool xpre = T <= DECODE_XPRE;

    // activations of the whole (small) batch are prepared while the expert
    // is looked up: thread -> (token, chunk)
    if (xpre) {
        for (int i = threadIdx.x; i < T * NK; i += NW * 64) {
            const int t = i / NK, c = i % NK;
            prep_chunk(x + (size_t)t * H + c * 32, &xp[t][c * 16], &xc[t][c]);
        }
    }
    if (wave == 0) {
        const uint8_t *bp = nullptr;
        int e = nth_active_expert(offsets, blobs, E, blockIdx.y, lane, &bp);
        // an expert without weights in the table, or one that `skip` lists
        // (done by an earlier launch), is left to another launch
        if (e >= 0 && (bp == nullptr || (skip != nullptr && skip[e] != nullptr)))
            e = -1;
        if (lane == 0) {
            s_e = e;
            s_blob = bp;
        }
    }
    __syncthreads();
    const int e = s_e;
    if (e < 0)
        return;
    const int p0 = offsets[e], p1 = offsets[e + 1];
    const uint8_t *blob = s_blob;
    const int IC = I / 32;                     // input chunks of the down rows

    // ---- issue every weight load of this workgroup up front
    const uint4_t *guq = reinterpret_cast<const uint4_t *>(blob + off_guq) +
                         ((size_t)slice * NK + (size_t)wave * CPW) * 64 + lane;
    uint4_t wq[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i)
        wq[i] = guq[(size_t)i * 64];
    const uint4_t *dqb = reinterpret_cast<const uint4_t *>(blob + off_dq);
    uint4_t dq[RBW];
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
        const int rb = wave * RBW + r;
        dq[r] = (rb < NRB) ? dqb[((size_t)rb * IC + slice) * 64 + lane] : uint4_t{0u, 0u, 0u, 0u};
    }
    const uint16_t *gus = reinterpret_cast<const uint16_t *>(blob + off_gus);
    const uint16_t *dsc = reinterpret_cast<const uint16_t *>(blob + off_ds);
    const int HG = H / g, IG = I / g;
    float sgu[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = wave * CPW + i;
        sgu[i] = h2f(gus[((size_t)slice * HG + (c * 32) / g) * 64 + lane]);
    }
    float sd[RBW];
#pragma unroll
    for (int r = 0; r < RBW; ++r) {
        const int rb = wave * RBW + r;
        sd[r] = (rb < NRB) ? h2f(dsc[((size_t)rb * IG + (slice * 32) / g) * 64 + lane]) : 0.0f;
    }

    for (int p = p0; p < p1; ++p) {
        const int t = perm[p] / k;
        int slot = t;
        if (!xpre) {
            slot = 0;
            for (int c = threadIdx.x; c < NK; c += NW * 64)
                prep_chunk(x + (size_t)t * H + c * 32, &xp[0][c * 16], &xc[0][c]);
            __syncthreads();
        }

        // gate/up rows (lane = row of the fused block), K split over waves
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = wave * CPW + i;
            const float d = dot_chunk(wq[i], &xp[slot][c * 16], xc[slot][c]);
            acc = fmaf(d, sgu[i], acc);
        }
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (wave == 0) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                v += red[w * 64 + lane];
            const float up = __shfl(v, (lane + 32) & 63, 64);
            // h for intermediate index lane (lanes < 32), rounded to fp16
            const f16 hq = (f16)(v / (1.0f + expf(-v)) * up);
            const bool odd = (lane >> 1) & 1;
            float cc = 0.0f;
            if (lane < 32) {
                reinterpret_cast<f16 *>(hp)[lane] = odd ? hq * (f16)0.0625f : hq;
                cc = (odd ? -72.0f : -1032.0f) * (float)hq;
            }
#pragma unroll
            for (int st = 16; st >= 1; st >>= 1)
                cc += __shfl_xor(cc, st, 64);
            if (lane == 0)
                hcorr = cc;
        }
        __syncthreads();

        // down strip: lane = output row, the 32 prepared h values from LDS
        float *yrow = y + ((size_t)slice * ntk + p) * H;
        const float hc = hcorr;
#pragma unroll
        for (int r = 0; r < RBW; ++r) {
            const int rb = wave * RBW + r;
            if (rb < NRB)
                yrow[rb * 64 + lane] = dot_chunk(dq[r], hp, hc) * sd[r];
        }
        __syncthreads();
    }
}

template <int H>
static void launch_decode_h(dim3 grid, hipStream_t s, const f16 *x, const int32_t *perm,
                            const int32_t *offsets, const uint8_t *const *blobs,
                            const uint8_t *const *skip, int I, int E, int k, int g, int ntk,
                            const DevLayout &L, float *y)
{
    constexpr int NW = (H >= 1024) ? 8 : 4;
    hipLaunchKernelGGL((ffn_decode_kernel<H, NW>), grid, dim3(NW * 64), 0, s, x, perm, offsets,
                       blobs, skip, I, E, k, g, ntk, L.gu_q, L.d_q, L.gu_s, L.d_s, y);
}

// skip (may be null): a device table of E pointers; experts with a non-null
// entry there are not computed (an earlier launch did them).  Experts with a
// null entry in `blobs` are not computed either.
int launch_ffn_decode(const void *x, const int32_t *perm, const int32_t *offsets,
                      const void *const *blobs, const void *const *skip, int T, int H, int I,
                      int E, int k, int g, float *y, hipStream_t s)
{
    const int ntk = T * k;
    if (ntk == 0)
        return MOE_OK;
    const DevLayout L = dev_layout(H, I, g);
    dim3 grid(I / 32, (unsigned)min(E, ntk));
    const f16 *xh = static_cast<const f16 *>(x);
    const uint8_t *const *b = reinterpret_cast<const uint8_t *const *>(blobs);
    const uint8_t *const *sk = reinterpret_cast<const uint8_t *const *>(skip);
    switch (H) {
    case 256: launch_decode_h<256>(grid, s, xh, perm, offsets, b, sk, I, E, k, g, ntk, L, y); break;
    case 512: launch_decode_h<512>(grid, s, xh, perm, offsets, b, sk, I, E, k, g, ntk, L, y); break;
    case 1024: launch_decode_h<1024>(grid, s, xh, perm, offsets, b, sk, I, E, k, g, ntk, L, y); break;
    case 2048: launch_decode_h<2048>(grid, s, xh, perm, offsets, b, sk, I, E, k, g, ntk, L, y); break;
    default: return set_error(MOE_EUNSUPPORTED, "decode kernel: H=%d not instantiated", H);
    }
    MOE_LAUNCH_CHECK("ffn_decode_kernel");
    return MOE_OK;
}

}  // namespace moe
