// k_route.hip -- router logits, softmax and top-k (K1), optionally fused with
// the token-to-expert permutation for batches that fit one workgroup.
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
// route_kernel (T <= 8, one workgroup): the TT tokens are staged in LDS;
// wave w computes experts w, w+NW, ... for all TT tokens, each router chunk
// loaded from global memory once and reused TT times.  A wave issues the
// loads of its next expert before the arithmetic of the current one.  Larger
// batches use route_logits_kernel + route_topk_kernel below.
#include "k_sort_common.h"

namespace moe {

template <int H, int TT, int NW>
__global__ __launch_bounds__(NW * 64) void route_kernel(
    const f16 *__restrict__ x, const f16 *__restrict__ wr, const float *__restrict__ bias,
    int T, int E, int k, unsigned flags, int32_t *__restrict__ idx_out, float *__restrict__ w_out)
{
    constexpr int NCH = H / 8;                // 8-element chunks of a row
    constexpr int NCL = (NCH + 63) / 64;      // chunks per lane
    extern __shared__ __align__(16) unsigned char smem[];
    f16 *xs = reinterpret_cast<f16 *>(smem);                                    // [TT][H]
    float *lg = reinterpret_cast<float *>(smem + (size_t)TT * H * sizeof(f16));  // [TT][E]
    const size_t tsb = topk_scratch_bytes(E);
    unsigned char *scr = smem + ((((size_t)TT * H * sizeof(f16) + (size_t)TT * E * sizeof(float)) + 15) & ~(size_t)15);   // [NW][tsb]
    Cand *sel = reinterpret_cast<Cand *>(scr + (size_t)NW * tsb);               // [NW][16]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * TT;
    const int nt = min(TT, T - t0);

    {
        constexpr int per_row = H / 8;
        const uint4_t *src = reinterpret_cast<const uint4_t *>(x);
        uint4_t *dst = reinterpret_cast<uint4_t *>(xs);
        for (int i = threadIdx.x; i < TT * per_row; i += NW * 64) {
            const int r = i / per_row;
            uint4_t v = {0u, 0u, 0u, 0u};
            if (r < nt)
                v = src[(size_t)(t0 + r) * per_row + (i % per_row)];
            dst[i] = v;
        }
    }

    uint4_t cur[NCL], nxt[NCL];
    auto load = [&](int e, uint4_t *dst) {
        const uint4_t *row = reinterpret_cast<const uint4_t *>(wr + (size_t)min(e, E - 1) * H);
#pragma unroll
        for (int m = 0; m < NCL; ++m) {
            const int c = lane + 64 * m;
            dst[m] = (e < E && c < NCH) ? row[c] : uint4_t{0u, 0u, 0u, 0u};
        }
    };
    load(wave, cur);
    __syncthreads();

    for (int e = wave; e < E; e += NW) {
        load(e + NW, nxt);
        float acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[tt] = 0.0f;
#pragma unroll
        for (int m = 0; m < NCL; ++m) {
            const int c = lane + 64 * m;
            if (c < NCH) {
                const half8_t wh = __builtin_bit_cast(half8_t, cur[m]);
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    const half8_t xh =
                        *reinterpret_cast<const half8_t *>(xs + (size_t)tt * H + c * 8);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[tt] = __builtin_fmaf((float)xh[i], (float)wh[i], acc[tt]);
                }
            }
        }
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float a = acc[tt];
            a = pinned_xor_sum(a, lane);
            if (bias)
                a = a + b;
            if (lane == 0)
                lg[tt * E + e] = a;
        }
#pragma unroll
        for (int m = 0; m < NCL; ++m)
            cur[m] = nxt[m];
    }
    __syncthreads();

    // top-k + softmax: wave w handles tokens w, w+NW, ...
    Cand *st = sel + wave * 16;
    for (int tt = wave; tt < nt; tt += NW) {
        const float *l = lg + tt * E;
        wave_topk(l, E, k, lane, st, scr + (size_t)wave * tsb);
        __builtin_amdgcn_wave_barrier();
        const float m = st[0].v;
        float part = 0.0f;
        for (int e = lane; e < E; e += 64)
            part += expf(l[e] - m);
        part = wave_sum_f32(part);   // softmax denominator (order fixed, not pinned)
        float p = 0.0f;
        if (lane < k)
            p = expf(st[lane].v - m) / part;
        if (flags & MOE_RENORM) {
            float ws = p;
            ws = wave_sum_f32(ws);
            p = p / ws;
        }
        if (lane < k) {
            const size_t t = (size_t)(t0 + tt);
            idx_out[t * k + lane] = st[lane].e;
            w_out[t * k + lane] = p;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Batches above 8 tokens: logits and top-k in two launches.
//
// route_logits_kernel: each wave computes an 8-token x 8-expert tile of
// logits.  Lane j owns partial j of all 64 logits (chunks c = j, j+64, ...,
// elements in order, acc = fma(x, w, acc) with exact fp16 products), reading
// its 16-byte slices of the 8 activation rows and the 8 router rows straight
// from memory (consecutive lanes read consecutive 16-byte slices of a row).
// The 64 x 64 partials then go through LDS so that lane l holds the 64
// partials of logit l and folds them in registers in the butterfly's order
// (a_j + a_(j+32), then +16, ... +1): the same additions, operand for operand,
// as the cross-lane butterfly, at one add per partial instead of a shuffle.
constexpr int RL_WAVES = 4;   // waves per workgroup, 8 experts each

template <int H>
__global__ __launch_bounds__(RL_WAVES * 64) void route_logits_kernel(
    const f16 *__restrict__ x, const f16 *__restrict__ wr, const float *__restrict__ bias,
    int T, int E, float *__restrict__ logits)
{
    constexpr int NCH = H / 8;                // 8-element chunks of a row
    constexpr int NCL = (NCH + 63) / 64;      // chunks per lane
    constexpr int RS = 68;                    // LDS row stride (floats) of the transposition
    __shared__ __align__(16) float tr[RL_WAVES][64 * RS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 8;
    const int e0 = (blockIdx.y * RL_WAVES + wave) * 8;

    float acc[8][8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[t][i] = 0.0f;
#pragma unroll
    for (int m = 0; m < NCL; ++m) {
        const int c = lane + 64 * m;
        if (c < NCH) {
            half8_t xv[8], wv[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int tt = min(t0 + t, T - 1);   // rows past T compute garbage, never stored
                xv[t] = *reinterpret_cast<const half8_t *>(x + (size_t)tt * H + c * 8);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ee = min(e0 + i, E - 1);
                wv[i] = *reinterpret_cast<const half8_t *>(wr + (size_t)ee * H + c * 8);
            }
#pragma unroll
            for (int el = 0; el < 8; ++el)
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[t][i] = __builtin_fmaf((float)xv[t][el], (float)wv[i][el], acc[t][i]);
        }
    }
    float *trw = tr[wave];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            trw[(t * 8 + i) * RS + lane] = acc[t][i];
    __builtin_amdgcn_wave_barrier();
    float a[64];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const float4_t v = *reinterpret_cast<const float4_t *>(trw + lane * RS + 4 * q);
        a[4 * q] = v[0];
        a[4 * q + 1] = v[1];
        a[4 * q + 2] = v[2];
        a[4 * q + 3] = v[3];
    }
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1)
#pragma unroll
        for (int j = 0; j < step; ++j)
            a[j] = a[j] + a[j + step];
    const int t = t0 + (lane >> 3), e = e0 + (lane & 7);
    if (t < T && e < E) {
        float l = a[0];
        if (bias)
            l = l + bias[e];
        logits[(size_t)t * E + e] = l;
    }
}

// route_topk_kernel: one wave per token over its E logits (rank-based top-k
// in 64-expert blocks, merge, softmax over all E in fp32, optional renorm).
constexpr int RT_WAVES = 4;

__global__ __launch_bounds__(RT_WAVES * 64) void route_topk_kernel(
    const float *__restrict__ logits, int T, int E, int k, unsigned flags,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // per wave: the token's logits (E floats, 16-byte aligned), then candidates
    const size_t lbytes = ((size_t)E * sizeof(float) + 15) & ~(size_t)15;
    const size_t tsb = topk_scratch_bytes(E);
    float *l = reinterpret_cast<float *>(smem + (size_t)wave * (lbytes + tsb + 16 * sizeof(Cand)));
    unsigned char *wc = reinterpret_cast<unsigned char *>(l) + lbytes;
    Cand *st = reinterpret_cast<Cand *>(wc + tsb);
    const int t = blockIdx.x * RT_WAVES + wave;
    if (t >= T)
        return;
    const float *lg = logits + (size_t)t * E;
    for (int e = lane; e < E; e += 64)   // every load of the row in flight at once
        l[e] = lg[e];
    __builtin_amdgcn_wave_barrier();
    wave_topk(l, E, k, lane, st, wc);
    __builtin_amdgcn_wave_barrier();
    const float m = st[0].v;
    float part = 0.0f;
    for (int e = lane; e < E; e += 64)
        part += expf(l[e] - m);
    part = wave_sum_f32(part);   // softmax denominator (order fixed, not pinned)
    float p = 0.0f;
    if (lane < k)
        p = expf(st[lane].v - m) / part;
    if (flags & MOE_RENORM) {
        float ws = p;
        ws = wave_sum_f32(ws);
        p = p / ws;
    }
    if (lane < k) {
        idx_out[(size_t)t * k + lane] = st[lane].e;
        w_out[(size_t)t * k + lane] = p;
    }
}

size_t route_batched_ws_bytes(int T, int E) { return (size_t)al256((int64_t)T * E * 4); }

// T > 8: logits into ws (T*E fp32), then top-k.
int launch_route_batched(const void *x, const void *wr, const float *bias, int T, int H, int E,
                         int k, unsigned flags, int32_t *idx, float *w, void *ws, hipStream_t s)
{
    float *lg = static_cast<float *>(ws);
    const f16 *xh = static_cast<const f16 *>(x), *wh = static_cast<const f16 *>(wr);
    const dim3 grid((T + 7) / 8, (E + 8 * RL_WAVES - 1) / (8 * RL_WAVES)), block(RL_WAVES * 64);
    switch (H) {
    case 256: hipLaunchKernelGGL(route_logits_kernel<256>, grid, block, 0, s, xh, wh, bias, T, E, lg); break;
    case 512: hipLaunchKernelGGL(route_logits_kernel<512>, grid, block, 0, s, xh, wh, bias, T, E, lg); break;
    case 1024: hipLaunchKernelGGL(route_logits_kernel<1024>, grid, block, 0, s, xh, wh, bias, T, E, lg); break;
    case 2048: hipLaunchKernelGGL(route_logits_kernel<2048>, grid, block, 0, s, xh, wh, bias, T, E, lg); break;
    default: return set_error(MOE_EUNSUPPORTED, "route: H=%d not instantiated", H);
    }
    MOE_LAUNCH_CHECK("route_logits_kernel");
    const size_t lds = (size_t)RT_WAVES * ((((size_t)E * sizeof(float) + 15) & ~(size_t)15) +
                                           topk_scratch_bytes(E) + 16 * sizeof(Cand));
    hipLaunchKernelGGL(route_topk_kernel, dim3((T + RT_WAVES - 1) / RT_WAVES),
                       dim3(RT_WAVES * 64), lds, s, lg, T, E, k, flags, idx, w);
    MOE_LAUNCH_CHECK("route_topk_kernel");
    return MOE_OK;
}

// Small batches (T <= 8) spread over many workgroups.  Workgroup g computes
// the logits of experts 4g..4g+3 (one wave each, every router load issued at
// once) for all T tokens and stores them to the workspace with agent-scope
// (write-through) stores; once they are acknowledged, one thread takes a
// ticket from an atomic counter (acquire-release at agent scope).  The
// workgroup holding the last ticket reads every logit back with agent-scope
// loads and does the top-k, the softmax and, when FUSE, the stable sort, then
// returns the counter to zero.  No workgroup ever waits for another.
// Experts (waves) per workgroup: 4 up to 128 experts; 16 above, so that 512
// experts take 32 workgroups and 32 ticket arrivals rather than 128 (one
// device-scope atomic on one address serialises at about 11 ns).
constexpr int rsplit_epw(bool bige) { return bige ? 16 : 4; }

template <int H, int TT, bool FUSE, bool BIGE>   // BIGE: E > 128
__global__ __launch_bounds__(rsplit_epw(BIGE) * 64) void route_split_kernel(
    const f16 *__restrict__ x, const f16 *__restrict__ wr, const float *__restrict__ bias,
    int T, int E, int k, unsigned flags, unsigned *ticket, float *ws_logits,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm,
    HostMirror hm)
{
    constexpr int RSPLIT_EPW = rsplit_epw(BIGE);
    constexpr int NCH = H / 8;
    constexpr int NCL = (NCH + 63) / 64;
    extern __shared__ __align__(16) unsigned char smem[];
    f16 *xs = reinterpret_cast<f16 *>(smem);   // [TT][H]; reused by the last group
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = blockIdx.x * RSPLIT_EPW + wave;

    uint4_t wv[NCL];
    {
        const uint4_t *row = reinterpret_cast<const uint4_t *>(wr + (size_t)min(e, E - 1) * H);
#pragma unroll
        for (int m = 0; m < NCL; ++m) {
            const int c = lane + 64 * m;
            wv[m] = (e < E && c < NCH) ? row[c] : uint4_t{0u, 0u, 0u, 0u};
        }
        const uint4_t *src = reinterpret_cast<const uint4_t *>(x);
        uint4_t *dst = reinterpret_cast<uint4_t *>(xs);
        for (int i = threadIdx.x; i < T * (H / 8); i += RSPLIT_EPW * 64)
            dst[i] = src[i];
    }
    __syncthreads();
    if (e < E) {
        float acc[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[tt] = 0.0f;
#pragma unroll
        for (int m = 0; m < NCL; ++m) {
            const int c = lane + 64 * m;
            if (c < NCH) {
                const half8_t wh = __builtin_bit_cast(half8_t, wv[m]);
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    if (tt < T) {
                        const half8_t xh =
                            *reinterpret_cast<const half8_t *>(xs + (size_t)tt * H + c * 8);
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            acc[tt] = __builtin_fmaf((float)xh[i], (float)wh[i], acc[tt]);
                    }
                }
            }
        }
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float a = acc[tt];
            a = pinned_xor_sum(a, lane);
            if (bias)
                a = a + b;
            if (lane == 0 && tt < T)
                __hip_atomic_store(ws_logits + tt * E + e, a, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's logit stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        // release: the workgroup's logit stores (ordered before it by the
        // barrier) are visible at agent scope before the ticket moves;
        // acquire: the last workgroup's reads below come after every other
        // workgroup's release
        const unsigned prev =
            __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last)
        return;

    if constexpr (FUSE && BIGE && TT == 1) {
        if (E <= RSPLIT_EPW * 64 && k <= 64) {
            // One token of 129..1024 experts: every wave of the workgroup,
            // thread e holding expert e.  A radix select over the unique
            // 64-bit selection keys (topk_key: the logit's order code, then
            // 0xFFFF - e; bits 16..31 are zero and skipped) finds the k-th
            // largest key four bits per round: each wave counts its
            // candidates per digit with 16 ballots, the counts meet in LDS
            // (double-buffered: one barrier per round), and every wave
            // derives the same bucket; the rounds stop once the bucket holds
            // exactly the keys still wanted.  The selected experts in id
            // order are the sort (position = selected experts of lower id);
            // wave 0 ranks the k selected keys and forms the softmax exactly
            // as the general path does (same terms, same order).
            int *hist = reinterpret_cast<int *>(smem);                           // [2][16][16]
            float *lgs = reinterpret_cast<float *>(smem + 2048);                 // [E <= 1024]
            int *wcnt = reinterpret_cast<int *>(smem + 2048 + 4096);             // [16]
            uint64_t *lkey = reinterpret_cast<uint64_t *>(smem + 2048 + 4096 + 64);   // [64]
            int *lidx = reinterpret_cast<int *>(lkey + 64);                      // [64]
            int *rke = lidx + 64;                                                // [64]
            const int e = threadIdx.x;
            const bool valid = e < E;
            const float lv = valid ? __hip_atomic_load(ws_logits + e, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT)
                                   : 0.0f;
            if (valid)
                lgs[e] = lv;
            if (threadIdx.x == 0)
                __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t key = valid ? topk_key(lv, e) : 0ull;
            uint64_t prefix = 0, pmask = 0;
            int r = k;
            for (int round = 0; round < 12; ++round) {
                const int sh = round < 8 ? 60 - 4 * round : 44 - 4 * round;   // 60..32, 12..0
                const bool cand = valid && (key & pmask) == prefix;
                const int dig = (int)((key >> sh) & 15u);
                int mycnt = 0;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int c = __popcll(__ballot(cand && dig == v));
                    mycnt = lane == v ? c : mycnt;
                }
                int *h = hist + (round & 1) * 256;
                if (lane < 16)
                    h[wave * 16 + lane] = mycnt;
                __syncthreads();
                int tot = 0;
                if (lane < 16)
                    for (int w = 0; w < RSPLIT_EPW; ++w)
                        tot += h[w * 16 + lane];
                int S = tot;   // lane v < 16: candidates with digit >= v
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) {
                    const int o = __shfl_down(S, off, 16);
                    S += lane + off < 16 ? o : 0;
                }
                const uint64_t bal = __ballot(lane < 16 && S >= r);
                const int d = 63 - __clzll((long long)bal);   // S_0 >= r: bal is never empty
                const int above = d < 15 ? __shfl(S, d + 1, 64) : 0;
                const int totd = __shfl(tot, d, 64);
                r -= above;
                prefix |= (uint64_t)d << sh;
                pmask |= (uint64_t)15 << sh;
                if (totd == r)
                    break;   // the same round in every wave
            }
            const bool sel = valid && key >= prefix;
            const uint64_t sb = __ballot(sel);
            const int below = __popcll(sb & ((1ull << lane) - 1ull));
            if (lane == 0)
                wcnt[wave] = __popcll(sb);
            __syncthreads();
            int pos = below;
            for (int w = 0; w < wave; ++w)
                pos += wcnt[w];
            if (valid) {
                counts[e] = sel ? 1 : 0;
                offsets[e] = pos;
            }
            if (e == E - 1)
                offsets[E] = k;
            if (sel) {
                lkey[pos] = key;
                lidx[pos] = e;
            }
            __syncthreads();
            if (wave != 0)
                return;
            // lane j < k: the selected expert at position j (id order), its rank
            const uint64_t mk = lane < k ? lkey[lane] : 0ull;
            int rank = 0;
            for (int j = 0; j < k; ++j)
                rank += lkey[j] > mk ? 1 : 0;
            if (lane < k) {
                rke[rank] = lidx[lane];
                perm[lane] = rank;
                inv_perm[rank] = lane;
            }
            __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
            const int er = lane < k ? rke[lane] : 0;   // lane j: the expert ranked j
            const float m = lgs[rke[0]];
            float part = 0.0f;
            for (int ee = lane; ee < E; ee += 64)
                part += expf(lgs[ee] - m);
            part = wave_sum_f32(part);   // softmax denominator (order fixed, not pinned)
            const float den = part;
            float pw = 0.0f;
            if (lane < k)
                pw = expf(lgs[er] - m) / den;
            if (flags & MOE_RENORM) {
                float ws = pw;
                ws = wave_sum_f32(ws);
                pw = pw / ws;
            }
            if (lane < k) {
                idx_out[lane] = er;
                w_out[lane] = pw;
            }
            return;
        }
    }

    if constexpr (FUSE && !BIGE && TT == 1) {
        if (E <= 64) {
            // One token of at most 64 experts: wave 0 alone, lane e holding
            // expert e, the selection and the sort in registers (same keys,
            // ranks and softmax terms as the general path below).
            if (wave != 0)
                return;
            const float l = lane < E ? __hip_atomic_load(ws_logits + lane, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)
                                     : 0.0f;
            if (lane == 0)
                __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            one_token_select(l, E, k, flags, reinterpret_cast<uint64_t *>(smem), idx_out, w_out,
                             counts, offsets, perm, inv_perm, lane, hm);
            return;
        }
    }

    const size_t tsb = topk_scratch_bytes(E);
    float *lg = reinterpret_cast<float *>(smem);                      // [T][E]
    unsigned char *scr = smem + ((((size_t)TT * E * sizeof(float)) + 15) & ~(size_t)15);   // [T][tsb]
    Cand *sel = reinterpret_cast<Cand *>(scr + (size_t)TT * tsb);     // [T][16]
    int *sidx = reinterpret_cast<int *>(sel + TT * 16);               // [T*k]
    int *cnt = sidx + TT * 16;                                        // [E]
    for (int i = threadIdx.x; i < T * E; i += RSPLIT_EPW * 64)
        lg[i] = __hip_atomic_load(ws_logits + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0)
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();

    // top-k, softmax and outputs: one wave per token
    for (int tt = wave; tt < T; tt += RSPLIT_EPW) {
        Cand *st = sel + tt * 16;
        wave_topk_t<BIGE ? 16 : 2>(lg + tt * E, E, k, lane, st, scr + (size_t)tt * tsb);
        __builtin_amdgcn_wave_barrier();
        const float m = st[0].v;
        float part = 0.0f;
        for (int ee = lane; ee < E; ee += 64)
            part += expf(lg[tt * E + ee] - m);
        part = wave_sum_f32(part);   // softmax denominator (order fixed, not pinned)
        const float den = part;
        float p = 0.0f;
        if (lane < k)
            p = expf(st[lane].v - m) / den;
        if (flags & MOE_RENORM) {
            float ws = p;
            ws = wave_sum_f32(ws);
            p = p / ws;
        }
        if (lane < k) {
            idx_out[(size_t)tt * k + lane] = st[lane].e;
            w_out[(size_t)tt * k + lane] = p;
            if (FUSE)
                sidx[tt * k + lane] = st[lane].e;
        }
    }
    if (FUSE) {
        lds_barrier();   // the sort reads sidx from LDS; the idx/w stores need not land first
        if (wave == 0) {
            const int n = T * k;
            if constexpr (!BIGE) {
                wave_small_sort(sidx, n, E, counts, offsets, perm, inv_perm, lane);
            } else {
                wave_count_scan(sidx, n, E, cnt, counts, offsets, lane);
                wave_stable_positions(sidx, n, perm, inv_perm, lane);
            }
        }
    }
}

size_t route_split_ws_bytes(int T, int E) { return 256 + (size_t)T * E * sizeof(float); }

// T <= 8; ws: zero-filled ticket (first 256 bytes) + T*E logits.
template <int H>
static int launch_route_split_h(const f16 *x, const f16 *wr, const float *bias, int T, int E,
                                int k, unsigned flags, int32_t *idx, float *w, int32_t *counts,
                                int32_t *offsets, int32_t *perm, int32_t *inv_perm, void *ws,
                                hipStream_t s, HostMirror hm = HostMirror{nullptr, nullptr, 0u})
{
    unsigned *ticket = static_cast<unsigned *>(ws);
    float *lg = reinterpret_cast<float *>(static_cast<char *>(ws) + 256);
    const int epw = rsplit_epw(E > 128);
    const dim3 grid((E + epw - 1) / epw), block(epw * 64);
    const size_t xb = (size_t)8 * H * sizeof(f16);
    const size_t lb = (size_t)8 * E * sizeof(float) + 16 + (size_t)8 * topk_scratch_bytes(E) +
                      (size_t)8 * 16 * sizeof(Cand) + (size_t)(8 * 16 + E) * sizeof(int);
    size_t lds = xb > lb ? xb : lb;
    if (lds < 8192)   // the one-token selection of more than 128 experts
        lds = 8192;
#define MOE_RSPLIT(TT)                                                                          \
    if (E > 128)                                                                                \
        hipLaunchKernelGGL((route_split_kernel<H, TT, true, true>), grid, block, lds, s, x, wr,  \
                           bias, T, E, k, flags, ticket, lg, idx, w, counts, offsets, perm,      \
                           inv_perm, hm);                                                        \
    else                                                                                        \
        hipLaunchKernelGGL((route_split_kernel<H, TT, true, false>), grid, block, lds, s, x, wr, \
                           bias, T, E, k, flags, ticket, lg, idx, w, counts, offsets, perm,      \
                           inv_perm, hm)
    if (T <= 1) MOE_RSPLIT(1);
    else if (T <= 2) MOE_RSPLIT(2);
    else if (T <= 4) MOE_RSPLIT(4);
    else MOE_RSPLIT(8);
#undef MOE_RSPLIT
    MOE_LAUNCH_CHECK("route_split_kernel");
    return MOE_OK;
}

int launch_route_split(const void *x, const void *wr, const float *bias, int T, int H, int E,
                       int k, unsigned flags, int32_t *idx, float *w, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv_perm, void *ws,
                       hipStream_t s)
{
    const f16 *xh = static_cast<const f16 *>(x), *wh = static_cast<const f16 *>(wr);
    switch (H) {
    case 256: return launch_route_split_h<256>(xh, wh, bias, T, E, k, flags, idx, w, counts,
                                               offsets, perm, inv_perm, ws, s);
    case 512: return launch_route_split_h<512>(xh, wh, bias, T, E, k, flags, idx, w, counts,
                                               offsets, perm, inv_perm, ws, s);
    case 1024: return launch_route_split_h<1024>(xh, wh, bias, T, E, k, flags, idx, w, counts,
                                                 offsets, perm, inv_perm, ws, s);
    case 2048: return launch_route_split_h<2048>(xh, wh, bias, T, E, k, flags, idx, w, counts,
                                                 offsets, perm, inv_perm, ws, s);
    default: return set_error(MOE_EUNSUPPORTED, "route: H=%d not instantiated", H);
    }
}

// One token of at most 64 experts with the routed ids also mirrored into
// host memory (the slot pool's wait for them): the fused route + permute of
// launch_route_split, bit for bit.  ws as for launch_route_split.
int launch_route_split_mirrored(const void *x, const void *wr, const float *bias, int H, int E,
                                int k, unsigned flags, int32_t *idx, float *w, int32_t *counts,
                                int32_t *offsets, int32_t *perm, int32_t *inv_perm, void *ws,
                                HostMirror hm, hipStream_t s)
{
    if (E > 64 || !hm.ids || !hm.flag)
        return set_error(MOE_EINVAL, "route: host mirror needs one token of at most 64 experts");
    const f16 *xh = static_cast<const f16 *>(x), *wh = static_cast<const f16 *>(wr);
    switch (H) {
    case 256: return launch_route_split_h<256>(xh, wh, bias, 1, E, k, flags, idx, w, counts,
                                               offsets, perm, inv_perm, ws, s, hm);
    case 512: return launch_route_split_h<512>(xh, wh, bias, 1, E, k, flags, idx, w, counts,
                                               offsets, perm, inv_perm, ws, s, hm);
    case 1024: return launch_route_split_h<1024>(xh, wh, bias, 1, E, k, flags, idx, w, counts,
                                                 offsets, perm, inv_perm, ws, s, hm);
    case 2048: return launch_route_split_h<2048>(xh, wh, bias, 1, E, k, flags, idx, w, counts,
                                                 offsets, perm, inv_perm, ws, s, hm);
    default: return set_error(MOE_EUNSUPPORTED, "route: H=%d not instantiated", H);
    }
}

template <int H>
static int launch_route_h(const f16 *x, const f16 *wr, const float *bias, int T, int E, int k,
                          unsigned flags, int32_t *idx, float *w, hipStream_t s)
{
    const size_t per_tok = (size_t)H * sizeof(f16) + (size_t)E * sizeof(float);
    auto lds_for = [&](int TT, int NW) {
        return (size_t)TT * per_tok + 16 + (size_t)NW * (topk_scratch_bytes(E) + 16 * sizeof(Cand));
    };
#define MOE_ROUTE_LAUNCH(TT, NW)                                                                 \
    hipLaunchKernelGGL((route_kernel<H, TT, NW>), dim3((T + TT - 1) / TT), dim3(NW * 64),        \
                       lds_for(TT, NW), s, x, wr, bias, T, E, k, flags, idx, w)
    // T <= 8 (larger batches take launch_route_batched): one workgroup of 16 waves
    if (T <= 1) MOE_ROUTE_LAUNCH(1, 16);
    else if (T <= 2) MOE_ROUTE_LAUNCH(2, 16);
    else if (T <= 4) MOE_ROUTE_LAUNCH(4, 16);
    else MOE_ROUTE_LAUNCH(8, 16);
#undef MOE_ROUTE_LAUNCH
    MOE_LAUNCH_CHECK("route_kernel");
    return MOE_OK;
}

int launch_route(const void *x, const void *wr, const float *bias, int T, int H, int E, int k,
                 unsigned flags, int32_t *idx, float *w, hipStream_t s)
{
    if (T == 0)
        return MOE_OK;
    const f16 *xh = static_cast<const f16 *>(x), *wh = static_cast<const f16 *>(wr);
    switch (H) {
    case 256: return launch_route_h<256>(xh, wh, bias, T, E, k, flags, idx, w, s);
    case 512: return launch_route_h<512>(xh, wh, bias, T, E, k, flags, idx, w, s);
    case 1024: return launch_route_h<1024>(xh, wh, bias, T, E, k, flags, idx, w, s);
    case 2048: return launch_route_h<2048>(xh, wh, bias, T, E, k, flags, idx, w, s);
    default: return set_error(MOE_EUNSUPPORTED, "route: H=%d not instantiated", H);
    }
}

}  // namespace moe
