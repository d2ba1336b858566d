// k_permute.hip -- token-to-expert grouping (K2).
//
// The pages' grouped executor computes the compact experts in groups
// (Horizon RunMap, "04 / Resultados"); this kernel produces that grouping:
// a stable counting sort of the flat index f = t*k + j by expert.
//   counts[E], offsets[E+1] (exclusive scan), perm[p] = f, inv_perm[f] = p,
// with f ascending inside each expert.  Integer work, one correct answer.
//
// Stability without atomics in the scatter: the flat range is cut into
// chunks of CH elements in order; chunk b's elements of expert e start at
// offsets[e] + (elements of e in chunks < b).  Inside a chunk one wave walks
// the elements 64 at a time; a lane's rank among equal keys of earlier lanes
// comes from ballots over the key bits, and a per-expert running counter in
// LDS advances by the group's multiplicity.
#include "k_sort_common.h"

namespace moe {

constexpr int PERM_CH = 512;     // elements per chunk in the multi-block path
constexpr int PERM_SMALL = 512;  // up to this many elements: one wave does everything
constexpr int PERM_BLOCK = 10240;   // up to this many (and E <= 1024): one workgroup
constexpr int PERM_BW = 16;         // its waves

// Whole sort in one wave (small T*k).
__global__ __launch_bounds__(64) void permute_small_kernel(
    const int32_t *__restrict__ idx, int n, int E, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm)
{
    extern __shared__ int cnt[];   // [E]
    wave_count_scan(idx, n, E, cnt, counts, offsets, threadIdx.x);
    wave_scatter(idx, 0, n, E, cnt, perm, inv_perm, threadIdx.x);
}

// Whole sort in one workgroup of 16 waves (moderate T*k, E <= 1024): the
// flat range is cut into 16 consecutive segments, one per wave.  Each wave
// counts its segment into its own LDS histogram; thread e then adds expert
// e's 16 counts, the workgroup scans them into offsets, and thread e turns
// its column of histograms into the running positions of expert e in each
// segment (offsets[e] + the segments before); each wave then scatters its
// segment in order -- the multi-block path's chunks, inside one launch.
__global__ __launch_bounds__(PERM_BW * 64) void permute_block_kernel(
    const int32_t *__restrict__ idx, int n, int E, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm)
{
    extern __shared__ int hw[];   // [PERM_BW][E]
    __shared__ int wsum[PERM_BW];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < PERM_BW * E; i += PERM_BW * 64)
        hw[i] = 0;
    __syncthreads();
    const int seg = ((n + PERM_BW - 1) / PERM_BW + 63) / 64 * 64;   // elements per wave
    const int f0 = min(n, w * seg), f1 = min(n, f0 + seg);
    int *h = hw + w * E;
    for (int b = f0; b < f1; b += 64 * WS_GROUPS) {   // keys loaded a batch at a time
        int keys[WS_GROUPS];
#pragma unroll
        for (int g = 0; g < WS_GROUPS; ++g) {
            const int f = b + 64 * g + lane;
            keys[g] = (f < f1) ? idx[f] : -1;
        }
#pragma unroll
        for (int g = 0; g < WS_GROUPS; ++g)
            if ((unsigned)keys[g] < (unsigned)E)
                atomicAdd(&h[keys[g]], 1);
    }
    __syncthreads();
    const int e = threadIdx.x;
    int hv[PERM_BW];
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < PERM_BW; ++ww) {
        hv[ww] = e < E ? hw[ww * E + e] : 0;
        c += hv[ww];
    }
    int incl = c;   // workgroup exclusive scan of c over e
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
        const int o = __shfl_up(incl, st, 64);
        if (lane >= st)
            incl += o;
    }
    if (lane == 63)
        wsum[w] = incl;
    __syncthreads();
    int pre = 0;
    for (int i = 0; i < w; ++i)
        pre += wsum[i];
    const int off = pre + incl - c;
    if (e < E) {
        counts[e] = c;
        offsets[e] = off;
        int run = off;
#pragma unroll
        for (int ww = 0; ww < PERM_BW; ++ww) {
            hw[ww * E + e] = run;
            run += hv[ww];
        }
    }
    if (e == 0)
        offsets[E] = n;
    __syncthreads();
    wave_scatter(idx, f0, f1, E, h, perm, inv_perm, lane);
}

// Phase 1: per-chunk histograms hist[b][E].
__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t *__restrict__ idx, int n,
                                                           int E, int32_t *__restrict__ hist)
{
    extern __shared__ int h[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        h[e] = 0;
    __syncthreads();
    const int f0 = b * PERM_CH, f1 = min(n, f0 + PERM_CH);
    static_assert(PERM_CH % 256 == 0, "whole rounds of 256 threads");
    int keys[PERM_CH / 256];
#pragma unroll
    for (int i = 0; i < PERM_CH / 256; ++i) {
        const int f = f0 + threadIdx.x + 256 * i;
        keys[i] = (f < f1) ? idx[f] : -1;
    }
#pragma unroll
    for (int i = 0; i < PERM_CH / 256; ++i)
        if ((unsigned)keys[i] < (unsigned)E)
            atomicAdd(&h[keys[i]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[(size_t)b * E + e] = h[e];
}

// Phase 2: counts, offsets and per-chunk bases (one block, thread per expert).
__global__ __launch_bounds__(1024) void permute_scan_kernel(
    const int32_t *__restrict__ hist, int nb, int E, int n, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ base)
{
    __shared__ int wsum[16];
    const int e = threadIdx.x;
    int c = 0;
    if (e < E) {
        int b = 0;
        for (; b + 8 <= nb; b += 8) {   // eight loads in flight per round
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = hist[(size_t)(b + i) * E + e];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                c += v[i];
        }
        for (; b < nb; ++b)
            c += hist[(size_t)b * E + e];
    }
    // block exclusive scan of c over e
    const int lane = e & 63, w = e >> 6;
    int incl = c;
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
        int o = __shfl_up(incl, st, 64);
        if (lane >= st)
            incl += o;
    }
    if (lane == 63)
        wsum[w] = incl;
    __syncthreads();
    int pre = 0;
    for (int i = 0; i < w; ++i)
        pre += wsum[i];
    const int off = pre + incl - c;
    if (e < E) {
        counts[e] = c;
        offsets[e] = off;
        int run = off;
        int b = 0;
        for (; b + 8 <= nb; b += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = hist[(size_t)(b + i) * E + e];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                base[(size_t)(b + i) * E + e] = run;
                run += v[i];
            }
        }
        for (; b < nb; ++b) {
            base[(size_t)b * E + e] = run;
            run += hist[(size_t)b * E + e];
        }
    }
    if (e == 0)
        offsets[E] = n;
}

// Phase 3: stable scatter, one wave per chunk.
__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t *__restrict__ idx, int n, int E, const int32_t *__restrict__ base,
    int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm)
{
    extern __shared__ int cnt[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 64)
        cnt[e] = base[(size_t)b * E + e];
    __syncthreads();
    const int f0 = b * PERM_CH, f1 = min(n, f0 + PERM_CH);
    wave_scatter(idx, f0, f1, E, cnt, perm, inv_perm, threadIdx.x);
}

static bool permute_one_block(int64_t n, int E) { return n <= PERM_BLOCK && E <= 1024; }

size_t permute_ws_bytes(int T, int k, int E)
{
    const int64_t n = (int64_t)T * k;
    if (n <= PERM_SMALL || permute_one_block(n, E))
        return 0;
    const int64_t nb = (n + PERM_CH - 1) / PERM_CH;
    return (size_t)(2 * nb * E * sizeof(int32_t));
}

int launch_permute(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets,
                   int32_t *perm, int32_t *inv_perm, void *ws, hipStream_t s)
{
    const int n = T * k;
    if (n <= PERM_SMALL) {
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(64), E * sizeof(int), s, idx, n,
                           E, counts, offsets, perm, inv_perm);
        MOE_LAUNCH_CHECK("permute_small_kernel");
        return MOE_OK;
    }
    if (permute_one_block(n, E)) {
        hipLaunchKernelGGL(permute_block_kernel, dim3(1), dim3(PERM_BW * 64),
                           (size_t)PERM_BW * E * sizeof(int), s, idx, n, E, counts, offsets, perm,
                           inv_perm);
        MOE_LAUNCH_CHECK("permute_block_kernel");
        return MOE_OK;
    }
    const int nb = (n + PERM_CH - 1) / PERM_CH;
    int32_t *hist = static_cast<int32_t *>(ws);
    int32_t *base = hist + (size_t)nb * E;
    hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(256), E * sizeof(int), s, idx, n, E,
                       hist);
    MOE_LAUNCH_CHECK("permute_hist_kernel");
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, s, hist, nb, E, n, counts,
                       offsets, base);
    MOE_LAUNCH_CHECK("permute_scan_kernel");
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(64), E * sizeof(int), s, idx, n, E,
                       base, perm, inv_perm);
    MOE_LAUNCH_CHECK("permute_scatter_kernel");
    return MOE_OK;
}

}  // namespace moe
