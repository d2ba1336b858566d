// k_combine_route.hip -- the combine of one decode layer fused with the
// router, top-k and sort of the next layer (one token, at most 64 experts).
//
// Two stacked layers meet at x_{l+1} = combine_l(...): the next layer's
// router needs every column of it, and the combine of a decode token is a
// few microseconds of latency-bound reads of the fp32 partials.  One launch
// does both.  In the pinned logit order (Horizon RunMap "08 / Comportamento
// do modelo": routing in FP32 with explicit roundings; the order itself is
// this library's reading) partial j of a logit accumulates the 8-column
// chunks j, j+64, j+128, ...  Block j (64 blocks, or H/8 when fewer) owns
// exactly those columns.  With the decode partials in partial-major column
// order (MOE_DTYPE_F32_PM) they lie side by side, so the block reads whole
// 128-byte lines of every partial row; in plain order it reads 32-byte
// pieces (correct, slower: four blocks share each line).  The block
//  1. combines its columns of x_{l+1} (combine_tile: the plain combine's
//     arithmetic, so the bits equal moe_combine's) and stores them;
//  2. with wave 0, lane e = expert e, accumulates partial j of every logit
//     from the fp16 x_{l+1} columns it just rounded, element by element in
//     chunk order, as the one-launch router does, and publishes the 64
//     partials as tagged words: one 64-bit store each, the value in the low
//     half and this call's tag in the high half, so a reader that sees the
//     tag sees the value (no acknowledgement, fence or ticket needed);
//  3. block 0 then polls the 64 x 64 tagged words until every tag is this
//     call's -- each of its four waves 16 partials of every logit, which
//     meet in LDS (one wave issuing all 64 loads per lane took 1.8 us from
//     the last store to the last tag seen, four waves 1.1 us) -- and wave 0
//     folds each logit's 64 partials in the butterfly order of the pinned
//     logit sum (pinned_fold64), adds the bias, selects, weights and sorts
//     as moe_route_permute does for one token (one_token_select), and
//     advances the call counter.
// Only block 0 waits, and only for blocks that never wait, so the wait ends
// whenever one more block can run beside it; a poll limit bounds it anyway.
// The tag is a quiet-NaN pattern carrying (call counter + 1) in its low 22
// bits: no finite value left in the region by another call can match it.
// The result is bit-identical to moe_combine followed by moe_route_permute.
#include "k_combine_tile.h"
#include "k_sort_common.h"

namespace moe {

constexpr int CR_MAX_POLLS = 1 << 20;   // far beyond any wait for co-running blocks

// Block j's i-th column: element i % 8 of chunk j + 64 (i / 8); in y at the
// same column (plain) or at its partial-major position 8 j q + i (PM).
template <bool PM>
struct PartialCols {
    int j, q;
    __device__ int col(int, int i) const { return 8 * (j + 64 * (i >> 3)) + (i & 7); }
    __device__ int y(int, int i) const { return PM ? 8 * j * q + i : col(0, i); }
};

// SEL = false: the partials are stored as plain fp32 into `part` ([64][64],
// partial j of expert e at j * 64 + e) and the launch ends there; the next
// layer's decode FFN folds and selects from them itself (ffn_decode_kernel
// with ROUTE), so no workgroup waits for another.
template <int H, bool GATED, bool PM, bool SEL>
__global__ __launch_bounds__(256) void combine_route_kernel(
    const float *__restrict__ y, int S, const int32_t *__restrict__ inv_perm,
    const float *__restrict__ w, const float *__restrict__ shared, const f16 *__restrict__ x,
    const f16 *__restrict__ wsg, const f16 *residual, int k, f16 *out,
    const f16 *__restrict__ wr, const float *__restrict__ bias, int E, int kn, unsigned flags,
    uint64_t *xchg, unsigned *calls, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ inv_perm_out, float *__restrict__ part)
{
    constexpr int NCH = H / 8;               // 8-column chunks
    constexpr int NCL = (NCH + 63) / 64;     // chunks per partial (all present: H % 512 == 0
                                             // or H = 256, where blocks j < 32 hold one)
    __shared__ CombineTileSmem sm[1];
    __shared__ __align__(16) f16 xs[32];
    __shared__ __align__(16) uint64_t keys[64];
    __shared__ float pl[SEL ? 64 : 1][64];   // block 0: the gathered logit partials

    const int j = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // the call counter, and the router chunks j + 64m of expert `lane` (lanes
    // past E read row E - 1; block 0 ignores them), requested first.  Every
    // wave issues them (only wave 0 uses them): a branch here would make the
    // compiler wait for them before the slice loads.
    const unsigned c = SEL ? __hip_atomic_load(calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0u;
    uint4_t wv[NCL];
    {
        const uint4_t *row =
            reinterpret_cast<const uint4_t *>(wr + (size_t)min(lane, E - 1) * H);
#pragma unroll
        for (int m = 0; m < NCL; ++m)
            wv[m] = row[j + 64 * m];
    }
    const PartialCols<PM> cols{j, NCL};
    const f16 o = combine_tile<GATED, 1>(y, S, inv_perm, w, shared, x, wsg, residual, 1, 0, H,
                                         k, 8 * NCL, cols, nullptr, sm, threadIdx.x);
    if (wave != 0 && j != 0)
        return;
    const unsigned tag = 0x7FC00000u | ((c + 1u) & 0x3FFFFFu);
    if (wave == 0) {
        if (lane < 8 * NCL) {
            xs[lane] = o;
            out[cols.col(0, lane)] = o;
        }
        __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
        float acc = 0.0f;
#pragma unroll
        for (int m = 0; m < NCL; ++m) {
            const half8_t xh = *reinterpret_cast<const half8_t *>(xs + 8 * m);
            const half8_t wh = __builtin_bit_cast(half8_t, wv[m]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc = __builtin_fmaf((float)xh[i], (float)wh[i], acc);
        }
        if constexpr (SEL)
            __hip_atomic_store(xchg + j * 64 + lane,
                               ((uint64_t)tag << 32) | __builtin_bit_cast(unsigned, acc),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            part[j * 64 + lane] = acc;
    }
    if (!SEL || j != 0)
        return;

    // block 0: wave w gathers partials 16w .. 16w+15 of every expert's logit
    // (lane e: expert e; partial jj >= gridDim.x has no chunk and is zero, as
    // in the one-launch router) with agent-scope loads until every tag is
    // this call's, and leaves them in LDS for wave 0
    const int nb = gridDim.x;
    float pv[16];
    for (int it = 0; it < CR_MAX_POLLS; ++it) {
        bool mine = true;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int jj = 16 * wave + i;
            const uint64_t q = __hip_atomic_load(xchg + min(jj, nb - 1) * 64 + lane,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pv[i] = jj < nb ? __builtin_bit_cast(float, (unsigned)q) : 0.0f;
            mine = mine && (unsigned)(q >> 32) == tag;
        }
        if (__ballot(!mine) == 0)
            break;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        pl[16 * wave + i][lane] = pv[i];
    __syncthreads();
    if (wave != 0)
        return;
    float p[64];
#pragma unroll
    for (int jj = 0; jj < 64; ++jj)
        p[jj] = pl[jj][lane];
    float l = pinned_fold64(p);
    if (bias)
        l = l + (lane < E ? bias[lane] : 0.0f);
    one_token_select(l, E, kn, flags, keys, idx_out, w_out, counts, offsets, perm, inv_perm_out,
                     lane);
    if (lane == 0)
        __hip_atomic_store(calls, tag & 0x3FFFFFu, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ws: [0, 256) the routers' ticket (not touched here), then 64 x 64 tagged
// words, then the call counter.
constexpr size_t CR_XCHG_OFF = 256;
constexpr size_t CR_CALLS_OFF = CR_XCHG_OFF + (size_t)64 * 64 * sizeof(uint64_t);
size_t combine_route_ws_bytes() { return CR_CALLS_OFF + 256; }

template <int H, bool GATED, bool PM>
static void launch_cr(const float *y, int S, const int32_t *inv_perm, const float *w,
                      const float *shared, const f16 *x, const f16 *wsg, const f16 *residual,
                      int k, f16 *out, const f16 *wr, const float *bias, int E, int kn,
                      unsigned flags, void *ws, int32_t *idx, float *wo, int32_t *counts,
                      int32_t *offsets, int32_t *perm, int32_t *inv_perm_out, float *part,
                      hipStream_t s)
{
    const int blocks = H / 8 < 64 ? H / 8 : 64;
    if (part) {
        hipLaunchKernelGGL((combine_route_kernel<H, GATED, PM, false>), dim3(blocks), dim3(256), 0,
                           s, y, S, inv_perm, w, shared, x, wsg, residual, k, out, wr, bias, E,
                           kn, flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, part);
        return;
    }
    char *base = static_cast<char *>(ws);
    uint64_t *xchg = reinterpret_cast<uint64_t *>(base + CR_XCHG_OFF);
    unsigned *calls = reinterpret_cast<unsigned *>(base + CR_CALLS_OFF);
    hipLaunchKernelGGL((combine_route_kernel<H, GATED, PM, true>), dim3(blocks), dim3(256), 0, s,
                       y, S, inv_perm, w, shared, x, wsg, residual, k, out, wr, bias, E, kn,
                       flags, xchg, calls, idx, wo, counts, offsets, perm, inv_perm_out, nullptr);
}

// T = 1, E <= 64, fp32 decode partials (pm: partial-major columns); the
// caller has checked the shapes.  part != null: store the next layer's logit
// partials there instead of routing (ws and the routing outputs unused).
int launch_combine_route(const float *y, bool pm, int S, const int32_t *inv_perm, const float *w,
                         const float *shared, const void *x, const void *gate_w,
                         const void *residual, int H, int k, void *out, const void *wr,
                         const float *bias, int E, int kn, unsigned flags, void *ws, int32_t *idx,
                         float *wo, int32_t *counts, int32_t *offsets, int32_t *perm,
                         int32_t *inv_perm_out, float *part, hipStream_t s)
{
    const f16 *xh = static_cast<const f16 *>(x), *gh = static_cast<const f16 *>(gate_w);
    const f16 *rh = static_cast<const f16 *>(residual), *wh = static_cast<const f16 *>(wr);
    f16 *oh = static_cast<f16 *>(out);
#define MOE_CR3(HH, G, P)                                                                       \
    launch_cr<HH, G, P>(y, S, inv_perm, w, shared, xh, gh, rh, k, oh, wh, bias, E, kn, flags,   \
                        ws, idx, wo, counts, offsets, perm, inv_perm_out, part, s)
#define MOE_CR(HH)                                                                              \
    if (gh) {                                                                                   \
        if (pm) MOE_CR3(HH, true, true);                                                        \
        else MOE_CR3(HH, true, false);                                                          \
    } else {                                                                                    \
        if (pm) MOE_CR3(HH, false, true);                                                       \
        else MOE_CR3(HH, false, false);                                                         \
    }
    switch (H) {
    case 256: MOE_CR(256) break;
    case 512: MOE_CR(512) break;
    case 1024: MOE_CR(1024) break;
    case 2048: MOE_CR(2048) break;
    default: return set_error(MOE_EUNSUPPORTED, "combine_route: H=%d not instantiated", H);
    }
#undef MOE_CR
#undef MOE_CR3
    MOE_LAUNCH_CHECK("combine_route_kernel");
    return MOE_OK;
}

// The 64 pinned-order partials of one token's router logits straight from
// an fp16 input row (the first layer of a stack, whose input no combine
// forms): block j, one wave, lane e = expert e, accumulates chunks j + 64 m
// of x against router row e element by element, as the combine above does
// from the columns it rounds, and stores partial j of every expert's logit
// at part[j * 64 + e].  Lanes past E repeat row E - 1 (never read back).
template <int H>
__global__ __launch_bounds__(64) void logit_partials_kernel(const f16 *__restrict__ x,
                                                            const f16 *__restrict__ wr, int E,
                                                            float *__restrict__ part)
{
    constexpr int NCH = H / 8;
    constexpr int NCL = (NCH + 63) / 64;
    const int j = blockIdx.x;
    const int lane = threadIdx.x;
    const uint4_t *row = reinterpret_cast<const uint4_t *>(wr + (size_t)min(lane, E - 1) * H);
    const uint4_t *xv = reinterpret_cast<const uint4_t *>(x);
    uint4_t wq[NCL], xq[NCL];
#pragma unroll
    for (int m = 0; m < NCL; ++m) {
        wq[m] = row[j + 64 * m];   // j + 64 m < NCH: the grid has min(64, NCH) blocks
        xq[m] = xv[j + 64 * m];
    }
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < NCL; ++m) {
        const half8_t xh = __builtin_bit_cast(half8_t, xq[m]);
        const half8_t wh = __builtin_bit_cast(half8_t, wq[m]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc = __builtin_fmaf((float)xh[i], (float)wh[i], acc);
    }
    part[j * 64 + lane] = acc;
}

// T = 1, E <= 64; the caller has checked the shapes and x's alignment.
int launch_logit_partials(const void *x, const void *wr, int H, int E, float *part, hipStream_t s)
{
    const f16 *xh = static_cast<const f16 *>(x), *wh = static_cast<const f16 *>(wr);
#define MOE_LP(HH)                                                                              \
    hipLaunchKernelGGL((logit_partials_kernel<HH>), dim3(HH / 8 < 64 ? HH / 8 : 64), dim3(64), \
                       0, s, xh, wh, E, part)
    switch (H) {
    case 256: MOE_LP(256); break;
    case 512: MOE_LP(512); break;
    case 1024: MOE_LP(1024); break;
    case 2048: MOE_LP(2048); break;
    default: return set_error(MOE_EUNSUPPORTED, "logit_partials: H=%d not instantiated", H);
    }
#undef MOE_LP
    MOE_LAUNCH_CHECK("logit_partials_kernel");
    return MOE_OK;
}

}  // namespace moe
