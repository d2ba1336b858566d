// k_combine.hip -- router-weighted combine (K6).
//
// Horizon RunMap "03 / Arquitetura": the experts' results return to the rest
// of the model, weighted by the router.  For token t, column c:
//   out = fp16_rne( sum_j w[t,j] * Y_j + s[t,c] + r[t,c] ),
//   Y_j = sum over slices of y[slice][inv_perm[t*k+j]][c],
// summed in fp32 in a fixed order (the slices in two contiguous halves, each
// in slice order, the halves then added; experts j ascending, then shared,
// then residual), so repeated runs give identical bits.
//
// Gated shared expert (the 60-expert top-4 model family of the Horizon RunMap
// technical preview, results table): the shared term becomes G_t * s[t,c] with
// G_t = sigmoid(x_t . wsg), the dot taken in fp32 by the block that needs it.
#include "k_combine_tile.h"

namespace moe {

// Shared-expert gate of one token: fp32 dot of x_t with wsg by the block's 256
// threads (8 columns per thread per pass), reduced over the block, then the
// sigmoid.  Every thread returns the same value.
__device__ inline float shared_gate_256(const f16 *__restrict__ xt, const f16 *__restrict__ wsg,
                                        int H, float *red)
{
    float a = 0.0f;
    for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
        const half8_t xv = *reinterpret_cast<const half8_t *>(xt + c);
        const half8_t wv = *reinterpret_cast<const half8_t *>(wsg + c);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            a = __builtin_fmaf((float)xv[m], (float)wv[m], a);
    }
#pragma unroll
    for (int off = 32; off; off >>= 1)
        a += __shfl_xor(a, off, 64);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = (red[0] + red[1]) + (red[2] + red[3]);
    return 1.0f / (1.0f + expf(-a));
}

// Decode partials: fp32 y [S][T*k][H], columns in plain or (PM)
// partial-major order.  Block = 32 consecutive y positions of one token
// (combine_tile); with PM the output columns are the positions' originals.
template <bool GATED, bool PM>
__global__ __launch_bounds__(256) void combine_slices_kernel(
    const float *__restrict__ y, int S, const int32_t *__restrict__ inv_perm,
    const float *__restrict__ w, const float *__restrict__ shared, const f16 *__restrict__ x,
    const f16 *__restrict__ wsg, const f16 *residual, int T, int H, int k, f16 *out)
{
    __shared__ CombineTileSmem sm[1];
    const int base = blockIdx.x * 32;
    if constexpr (PM)
        combine_tile<GATED, 1>(y, S, inv_perm, w, shared, x, wsg, residual, T, blockIdx.y, H, k,
                               min(32, H - base), PmCols{base, H}, out, sm, threadIdx.x);
    else
        combine_tile<GATED, 1>(y, S, inv_perm, w, shared, x, wsg, residual, T, blockIdx.y, H, k,
                               min(32, H - base), ContigCols{base}, out, sm, threadIdx.x);
}

// 8 consecutive columns of one y row, loaded as one (fp16) or two (fp32)
// 16-byte vectors; converted only when summed, so a thread's loads of all k
// rows can be in flight together.
template <typename YT>
struct Row8;
template <>
struct Row8<f16> {
    half8_t v;
    __device__ void load(const f16 *p) { v = *reinterpret_cast<const half8_t *>(p); }
    __device__ float at(int m) const { return (float)v[m]; }
};
template <>
struct Row8<float> {
    float4_t a, b;
    __device__ void load(const float *p)
    {
        a = reinterpret_cast<const float4_t *>(p)[0];
        b = reinterpret_cast<const float4_t *>(p)[1];
    }
    __device__ float at(int m) const { return m < 4 ? a[m] : b[m - 4]; }
};

// Adds sum_j w[t,j] * y[inv_perm[t*k+j]][c0..c0+8) to acc in j order.  KMAX
// >= k: every index, weight and row load is issued before the first add (at
// clamped j, so none is conditional); rows past k are loaded again, not added.
template <typename YT, int KMAX>
__device__ __forceinline__ void routed_sum8(const YT *__restrict__ y,
                                            const int32_t *__restrict__ inv_perm,
                                            const float *__restrict__ w, int t, int H, int k,
                                            int c0, float (&acc)[8])
{
    int32_t pj[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int jj = min(j, k - 1);
        pj[j] = inv_perm ? inv_perm[(size_t)t * k + jj] : t * k + jj;   // NULL: token order
        wj[j] = w[(size_t)t * k + jj];
    }
    Row8<YT> r[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        r[j].load(y + (size_t)pj[j] * H + c0);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (j < k) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
                acc[m] += wj[j] * r[j].at(m);
        }
}

// One slice (fp16 or fp32 y [T*k][H]): thread per (token, 8 columns).
template <typename YT, int KMAX>
__global__ __launch_bounds__(256) void combine_rows_kernel(
    const YT *__restrict__ y, const int32_t *__restrict__ inv_perm, const float *__restrict__ w,
    const float *__restrict__ shared, const f16 *residual, int T, int H, int k, f16 *out)
{
    const int per_row = H / 8;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * per_row)
        return;
    const int t = (int)(i / per_row);
    const int c0 = (int)(i % per_row) * 8;
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        acc[m] = 0.0f;
    routed_sum8<YT, KMAX>(y, inv_perm, w, t, H, k, c0, acc);
    if (shared) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[m] += shared[(size_t)t * H + c0 + m];
    }
    if (residual) {
        const half8_t r = *reinterpret_cast<const half8_t *>(residual + (size_t)t * H + c0);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[m] += (float)r[m];
    }
    half8_t o;
#pragma unroll
    for (int m = 0; m < 8; ++m)
        o[m] = (f16)acc[m];
    *reinterpret_cast<half8_t *>(out + (size_t)t * H + c0) = o;
}

// One slice with the gated shared term: one block per token; the block first
// forms the token's gate, then each thread handles 8 columns per pass.
template <typename YT, int KMAX>
__global__ __launch_bounds__(256) void combine_rows_gated_kernel(
    const YT *__restrict__ y, const int32_t *__restrict__ inv_perm, const float *__restrict__ w,
    const float *__restrict__ shared, const f16 *__restrict__ x, const f16 *__restrict__ wsg,
    const f16 *residual, int H, int k, f16 *out)
{
    __shared__ float red[4];
    const int t = blockIdx.x;
    const float gate = shared_gate_256(x + (size_t)t * H, wsg, H, red);
    for (int c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
        float acc[8];
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[m] = 0.0f;
        routed_sum8<YT, KMAX>(y, inv_perm, w, t, H, k, c0, acc);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[m] += gate * shared[(size_t)t * H + c0 + m];
        if (residual) {
            const half8_t r = *reinterpret_cast<const half8_t *>(residual + (size_t)t * H + c0);
#pragma unroll
            for (int m = 0; m < 8; ++m)
                acc[m] += (float)r[m];
        }
        half8_t o;
#pragma unroll
        for (int m = 0; m < 8; ++m)
            o[m] = (f16)acc[m];
        *reinterpret_cast<half8_t *>(out + (size_t)t * H + c0) = o;
    }
}

template <typename YT, int KMAX, bool GATED>
static int launch_rows(const YT *y, const int32_t *inv_perm, const float *w, const float *shared,
                       const f16 *x, const f16 *gw, const f16 *res, int T, int H, int k, f16 *o,
                       hipStream_t s)
{
    if constexpr (GATED) {
        hipLaunchKernelGGL((combine_rows_gated_kernel<YT, KMAX>), dim3(T), dim3(256), 0, s, y,
                           inv_perm, w, shared, x, gw, res, H, k, o);
        MOE_LAUNCH_CHECK("combine_rows_gated_kernel");
    } else {
        const size_t n = (size_t)T * (H / 8);
        hipLaunchKernelGGL((combine_rows_kernel<YT, KMAX>), dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, s, y, inv_perm, w, shared, res, T, H, k, o);
        MOE_LAUNCH_CHECK("combine_rows_kernel");
    }
    return MOE_OK;
}

template <typename YT, bool GATED>
static int launch_rows_k(const YT *y, const int32_t *inv_perm, const float *w, const float *shared,
                         const f16 *x, const f16 *gw, const f16 *res, int T, int H, int k, f16 *o,
                         hipStream_t s)
{
    if (k <= 4)
        return launch_rows<YT, 4, GATED>(y, inv_perm, w, shared, x, gw, res, T, H, k, o, s);
    if (k <= 8)
        return launch_rows<YT, 8, GATED>(y, inv_perm, w, shared, x, gw, res, T, H, k, o, s);
    if (k <= 12)
        return launch_rows<YT, 12, GATED>(y, inv_perm, w, shared, x, gw, res, T, H, k, o, s);
    return launch_rows<YT, 16, GATED>(y, inv_perm, w, shared, x, gw, res, T, H, k, o, s);
}

int launch_combine(const void *y, int y_dtype, int S, const int32_t *inv_perm, const float *w,
                   const float *shared, const void *x_f16, const void *gate_w_f16,
                   const void *residual, int T, int H, int k, void *out, hipStream_t s)
{
    if (T == 0)
        return MOE_OK;
    const f16 *res = static_cast<const f16 *>(residual);
    const f16 *xh = static_cast<const f16 *>(x_f16);
    const f16 *gw = static_cast<const f16 *>(gate_w_f16);
    const bool gated = gw != nullptr;
    f16 *o = static_cast<f16 *>(out);
    if ((y_dtype == MOE_DTYPE_F32 && S > 1) || y_dtype == MOE_DTYPE_F32_PM) {
        dim3 grid((H + 31) / 32, T);
        const float *yf = static_cast<const float *>(y);
#define MOE_SLICES(G, P)                                                                         \
    hipLaunchKernelGGL((combine_slices_kernel<G, P>), grid, dim3(256), 0, s, yf, S, inv_perm, w, \
                       shared, xh, gw, res, T, H, k, o)
        const bool pm = y_dtype == MOE_DTYPE_F32_PM;
        if (gated) {
            if (pm) MOE_SLICES(true, true);
            else MOE_SLICES(true, false);
        } else {
            if (pm) MOE_SLICES(false, true);
            else MOE_SLICES(false, false);
        }
#undef MOE_SLICES
        MOE_LAUNCH_CHECK("combine_slices_kernel");
        return MOE_OK;
    }
    if (gated) {
        if (y_dtype == MOE_DTYPE_F32)
            return launch_rows_k<float, true>(static_cast<const float *>(y), inv_perm, w, shared,
                                              xh, gw, res, T, H, k, o, s);
        return launch_rows_k<f16, true>(static_cast<const f16 *>(y), inv_perm, w, shared, xh, gw,
                                        res, T, H, k, o, s);
    }
    if (y_dtype == MOE_DTYPE_F32)
        return launch_rows_k<float, false>(static_cast<const float *>(y), inv_perm, w, shared,
                                           xh, gw, res, T, H, k, o, s);
    return launch_rows_k<f16, false>(static_cast<const f16 *>(y), inv_perm, w, shared, xh, gw,
                                     res, T, H, k, o, s);
}

}  // namespace moe
