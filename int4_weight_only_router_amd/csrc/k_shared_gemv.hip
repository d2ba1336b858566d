// k_shared_gemv.hip -- the shared FP16 expert at small T: a GEMV pair
// (gate/up + SwiGLU, then down) straight from the row-major fp16 weights.
//
// Horizon RunMap "03 / Arquitetura": the non-routed parts of the model stay
// in FP16 outside the INT4 compression.
#include "moe_common.h"

namespace moe {

// FP16 GEMV pair for the shared expert at small T (weights row-major fp16,
// the layout the caller hands over).  One wave per output row, lanes along K
// with 16-byte loads, every token's dot product from the same weight
// registers, a DPP wave sum at the end.  A pass covers U chunks of 8 K per
// lane and issues all of its loads (weights and the tokens' K slices, at
// clamped indices, so none is conditional) before any arithmetic: a long row
// costs a few round trips instead of one per chunk.
//   SW=1: h[t][r] = fp16(silu(Wg[r].x_t) * (Wu[r].x_t)), r < R
//   SW=0: out[t][r] = W[r].in_t (fp32), r < R
constexpr int GEMV_WAVES = 4;

template <int T_MAX, int U, bool SW>
__global__ __launch_bounds__(GEMV_WAVES * 64) void gemv_f16_kernel(
    const f16 *__restrict__ in, const f16 *__restrict__ wa, const f16 *__restrict__ wb, int T,
    int R, int K, f16 *__restrict__ hout, float *__restrict__ fout)
{
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * GEMV_WAVES + (threadIdx.x >> 6);
    if (r >= R)
        return;
    const int nch = K / 8;
    const int npass = (nch + 64 * U - 1) / (64 * U);
    const uint4_t *ra = reinterpret_cast<const uint4_t *>(wa + (size_t)r * K);
    const uint4_t *rb = SW ? reinterpret_cast<const uint4_t *>(wb + (size_t)r * K) : nullptr;
    const uint4_t *xr[T_MAX];
#pragma unroll
    for (int t = 0; t < T_MAX; ++t)
        xr[t] = reinterpret_cast<const uint4_t *>(in + (size_t)min(t, T - 1) * K);
    float aa[T_MAX], bb[T_MAX];
#pragma unroll
    for (int t = 0; t < T_MAX; ++t) {
        aa[t] = 0.0f;
        bb[t] = 0.0f;
    }
    for (int pass = 0; pass < npass; ++pass) {
        const int c0 = pass * 64 * U + lane;
        uint4_t va[U], vb[U], xv[T_MAX][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = min(c0 + 64 * u, nch - 1);
            va[u] = ldg_nt(ra + c);   // weights: read once per call
            if constexpr (SW)
                vb[u] = ldg_nt(rb + c);
#pragma unroll
            for (int t = 0; t < T_MAX; ++t)
                xv[t][u] = xr[t][c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = c0 + 64 * u < nch;
            const uint4_t z = {0u, 0u, 0u, 0u};
            const half8_t a8 = __builtin_bit_cast(half8_t, ok ? va[u] : z);
            half8_t b8 = {};
            if constexpr (SW)
                b8 = __builtin_bit_cast(half8_t, ok ? vb[u] : z);
#pragma unroll
            for (int t = 0; t < T_MAX; ++t) {
                const half8_t x8 = __builtin_bit_cast(half8_t, xv[t][u]);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const half2_t xp = {x8[2 * m], x8[2 * m + 1]};
                    const half2_t ap = {a8[2 * m], a8[2 * m + 1]};
                    aa[t] = dot2(ap, xp, aa[t]);
                    if constexpr (SW) {
                        const half2_t bp = {b8[2 * m], b8[2 * m + 1]};
                        bb[t] = dot2(bp, xp, bb[t]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T_MAX; ++t) {
        if (t >= T)
            continue;
        const float a = wave_sum_f32(aa[t]);
        const float b = SW ? wave_sum_f32(bb[t]) : 0.0f;
        if (lane == 0) {
            if constexpr (SW)
                hout[(size_t)t * R + r] = (f16)(a / (1.0f + expf(-a)) * b);
            else
                fout[(size_t)t * R + r] = a;
        }
    }
}

// Chunks per lane and pass: no more than a row has (a clamped duplicate load
// still costs an instruction), at most UMAX (registers).
template <int UMAX>
static int gemv_u(int K)
{
    const int per_lane = (K / 8 + 63) / 64;
    int u = 2;
    while (u < UMAX && u < per_lane)
        u *= 2;
    return u;
}

template <int T_MAX, int U, bool SW>
static void launch_gemv(int R, hipStream_t s, const f16 *in, const f16 *wa, const f16 *wb, int T,
                        int K, f16 *h, float *out)
{
    hipLaunchKernelGGL((gemv_f16_kernel<T_MAX, U, SW>), dim3((R + GEMV_WAVES - 1) / GEMV_WAVES),
                       dim3(GEMV_WAVES * 64), 0, s, in, wa, wb, T, R, K, h, out);
}

template <int T_MAX, int UMAX, bool SW>
static void launch_gemv_u(int R, hipStream_t s, const f16 *in, const f16 *wa, const f16 *wb, int T,
                          int K, f16 *h, float *out)
{
    const int u = gemv_u<UMAX>(K);
    if (u <= 2)
        launch_gemv<T_MAX, (UMAX < 2 ? UMAX : 2), SW>(R, s, in, wa, wb, T, K, h, out);
    else if (u <= 4)
        launch_gemv<T_MAX, (UMAX < 4 ? UMAX : 4), SW>(R, s, in, wa, wb, T, K, h, out);
    else
        launch_gemv<T_MAX, UMAX, SW>(R, s, in, wa, wb, T, K, h, out);
}

template <int T_MAX, int U>
static int launch_gemv_pair(const void *x, const void *wg, const void *wu, const void *wd, int T,
                            int H, int Is, float *out, f16 *h, hipStream_t s)
{
    launch_gemv_u<T_MAX, U, true>(Is, s, (const f16 *)x, (const f16 *)wg, (const f16 *)wu, T, H, h,
                                  (float *)nullptr);
    MOE_LAUNCH_CHECK("gemv_f16_kernel(gate/up)");
    launch_gemv_u<T_MAX, U, false>(H, s, (const f16 *)h, (const f16 *)wd, (const f16 *)nullptr, T,
                                   Is, (f16 *)nullptr, out);
    MOE_LAUNCH_CHECK("gemv_f16_kernel(down)");
    return MOE_OK;
}

// Small T: a weight row is read once and dotted with every token's row
// (accumulators for up to T_MAX tokens per lane).
int launch_shared_gemv(const void *x, const void *wg, const void *wu, const void *wd, int T,
                       int H, int Is, float *out, void *ws, hipStream_t s)
{
    f16 *h = shared_ffn_h(ws);   // [T][Is]
    if (T <= 1)
        return launch_gemv_pair<1, 8>(x, wg, wu, wd, T, H, Is, out, h, s);
    if (T <= 2)
        return launch_gemv_pair<2, 8>(x, wg, wu, wd, T, H, Is, out, h, s);
    if (T <= 4)
        return launch_gemv_pair<4, 4>(x, wg, wu, wd, T, H, Is, out, h, s);
    if (T <= 8)
        return launch_gemv_pair<8, 2>(x, wg, wu, wd, T, H, Is, out, h, s);
    return set_error(MOE_EUNSUPPORTED, "shared GEMV: T=%d > 8", T);
}

}  // namespace moe
