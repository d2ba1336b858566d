// k_route.hip -- router logits, softmax and top-k (K1).
//
// Horizon RunMap, "03 / Arquitetura": the router selects the experts that
// work on each token; "08 / Comportamento do modelo": routing stays outside
// INT4 and accumulation is FP32 with explicit roundings.  The pages leave the
// rest open; this kernel fixes it as follows.
//  * Logit l[t,e] = sum_h x[t,h] Wr[e,h] in fp32 in a pinned order: chunk c
//    (8 consecutive h) is accumulated, element by element, into partial
//    number (c mod 64), chunks in increasing c; the 64 partials are combined
//    by an xor butterfly with strides 32,16,8,4,2,1.  Partial j lives in lane
//    j of the wave that owns (t, e), so the butterfly is a lane shuffle.
//    fp16 x fp16 products are exact in fp32, hence fma and mul+add agree and
//    the logits are reproducible bit for bit.
//  * Optional fp32 bias added after the dot product.
//  * Top-k by (logit desc, expert asc); softmax over all E logits taken at the
//    chosen experts; optional renormalisation over the k chosen.
//
// Work split: a workgroup of 4 waves owns TT tokens (x tile staged in LDS);
// wave w computes experts w, w+4, ... for all TT tokens, so each router
// chunk loaded from global memory is reused TT times.
#include "moe_common.h"

namespace moe {

constexpr int ROUTE_WAVES = 4;

template <int TT>
__global__ __launch_bounds__(ROUTE_WAVES * 64) void route_kernel(
    const f16 *__restrict__ x, const f16 *__restrict__ wr, const float *__restrict__ bias,
    int T, int H, int E, int k, unsigned flags, int32_t *__restrict__ idx_out,
    float *__restrict__ w_out)
{
    extern __shared__ __align__(16) unsigned char smem[];
    f16 *xs = reinterpret_cast<f16 *>(smem);                                  // [TT][H]
    float *lg = reinterpret_cast<float *>(smem + (size_t)TT * H * sizeof(f16));  // [TT][E]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * TT;
    const int nt = min(TT, T - t0);

    // x tile -> LDS (16-byte pieces); rows past T are zero
    {
        const int per_row = H / 8;
        const uint4_t *src = reinterpret_cast<const uint4_t *>(x);
        uint4_t *dst = reinterpret_cast<uint4_t *>(xs);
        for (int i = threadIdx.x; i < TT * per_row; i += blockDim.x) {
            int r = i / per_row;
            uint4_t v = {0u, 0u, 0u, 0u};
            if (r < nt)
                v = src[(size_t)(t0 + r) * per_row + (i % per_row)];
            dst[i] = v;
        }
    }
    __syncthreads();

    const int nchunk = H / 8;
    for (int e = wave; e < E; e += ROUTE_WAVES) {
        float acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[tt] = 0.0f;
        const uint4_t *wrow = reinterpret_cast<const uint4_t *>(wr + (size_t)e * H);
        for (int c = lane; c < nchunk; c += 64) {
            uint4_t wv = wrow[c];
            half8_t wh = __builtin_bit_cast(half8_t, wv);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                half8_t xh = *reinterpret_cast<const half8_t *>(xs + (size_t)tt * H + c * 8);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[tt] = acc[tt] + (float)xh[i] * (float)wh[i];
            }
        }
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float a = acc[tt];
#pragma unroll
            for (int st = 32; st >= 1; st >>= 1)
                a = a + __shfl_xor(a, st, 64);
            if (bias)
                a = a + b;
            if (lane == 0)
                lg[tt * E + e] = a;
        }
    }
    __syncthreads();

    // top-k + softmax: wave w handles tokens w, w+4, ...
    for (int tt = wave; tt < nt; tt += ROUTE_WAVES) {
        const float *l = lg + tt * E;
        // each lane scans its experts e = lane + 64 m; "taken" bits per lane
        uint32_t taken = 0u;   // bit m set when expert lane+64m chosen (E <= 2048)
        float vsel[16];
        int esel[16];
        for (int j = 0; j < k; ++j) {
            float bv = 0.0f;
            int be = 0x7fffffff;
            for (int m = 0, e = lane; e < E; ++m, e += 64) {
                if (taken & (1u << m))
                    continue;
                float v = l[e];
                if (be == 0x7fffffff || v > bv) {   // ascending e: ties keep lower index
                    bv = v;
                    be = e;
                }
            }
            // wave argmax with lower-index tie-break
#pragma unroll
            for (int st = 32; st >= 1; st >>= 1) {
                float ov = __shfl_xor(bv, st, 64);
                int oe = __shfl_xor(be, st, 64);
                bool take = (oe != 0x7fffffff) &&
                            (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
                if (take) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be & 63) == lane)
                taken |= 1u << (be >> 6);
            vsel[j] = bv;
            esel[j] = be;
        }
        // softmax over all E (fp32), max = best logit
        const float m = vsel[0];
        float part = 0.0f;
        for (int e = lane; e < E; e += 64)
            part += expf(l[e] - m);
#pragma unroll
        for (int st = 32; st >= 1; st >>= 1)
            part += __shfl_xor(part, st, 64);
        const float den = part;
        float wsum = 0.0f;
        for (int j = 0; j < k; ++j)
            wsum += expf(vsel[j] - m) / den;
        if (lane == 0) {
            const size_t t = (size_t)(t0 + tt);
            for (int j = 0; j < k; ++j) {
                float p = expf(vsel[j] - m) / den;
                if (flags & MOE_RENORM)
                    p = p / wsum;
                idx_out[t * k + j] = esel[j];
                w_out[t * k + j] = p;
            }
        }
    }
}

int launch_route(const void *x, const void *wr, const float *bias, int T, int H, int E, int k,
                 unsigned flags, int32_t *idx, float *w, hipStream_t s)
{
    if (T == 0)
        return MOE_OK;
    // tokens per workgroup: 8 for large T, fewer if the tile would exceed the
    // default 64 KB of dynamic LDS
    const size_t per_tok = (size_t)H * sizeof(f16) + (size_t)E * sizeof(float);
    int TT = (T >= 64) ? 8 : 1;
    while (TT > 1 && TT * per_tok > 65536)
        TT >>= 1;
    const size_t lds = TT * per_tok;
    dim3 grid((T + TT - 1) / TT), block(ROUTE_WAVES * 64);
    const f16 *xh = static_cast<const f16 *>(x), *wh = static_cast<const f16 *>(wr);
    switch (TT) {
    case 8: hipLaunchKernelGGL(route_kernel<8>, grid, block, lds, s, xh, wh, bias, T, H, E, k,
                               flags, idx, w); break;
    case 4: hipLaunchKernelGGL(route_kernel<4>, grid, block, lds, s, xh, wh, bias, T, H, E, k,
                               flags, idx, w); break;
    case 2: hipLaunchKernelGGL(route_kernel<2>, grid, block, lds, s, xh, wh, bias, T, H, E, k,
                               flags, idx, w); break;
    default: hipLaunchKernelGGL(route_kernel<1>, grid, block, lds, s, xh, wh, bias, T, H, E, k,
                                flags, idx, w); break;
    }
    MOE_LAUNCH_CHECK("route_kernel");
    return MOE_OK;
}

}  // namespace moe
