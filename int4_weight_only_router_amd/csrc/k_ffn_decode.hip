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
// workgroup writes an fp32 partial y for its slice (at the row's sorted
// position, or at t*k + j with MOE_Y_TOKEN_ORDER; each column at its
// partial-major position with MOE_Y_PARTIAL_ORDER); moe_combine adds the
// slices in order.  Each wave keeps a few weight chunks in flight and
// computes each chunk as it lands (schedule notes at the kernel).
#include "k_decode_frag.h"
#include "k_sort_common.h"

#include <type_traits>

namespace moe {

// Finds the a-th expert (in id order) with at least one routed row; -1 if
// none.  The blob pointer and the expert's row range are fetched in the same
// sweep as the offsets, so all three are known one memory round trip after
// entry.  Every wave runs it on its own (the same addresses: one trip to
// memory, the rest hit the caches), so no wave waits on a barrier before it
// issues its weight loads.
__device__ __forceinline__ int nth_active_expert(const int32_t *__restrict__ offsets,
                                                 const uint8_t *const *__restrict__ blobs, int E,
                                                 int a, int lane, const uint8_t **blob_out,
                                                 int *p0_out, int *p1_out)
{
    int seen = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const bool inb = e < E;
        const int o0 = inb ? ldg(offsets + e) : 0;
        const int o1 = inb ? ldg(offsets + e + 1) : 0;
        const uint8_t *bp = inb ? ldg(blobs + e) : nullptr;
        const bool act = o1 > o0;
        const uint64_t m = __ballot(act);
        const int n = __popcll(m);
        if (seen + n > a) {
            const int r = a - seen;
            const int rank = __popcll(m & ((1ull << lane) - 1ull));
            const uint64_t hit = __ballot(act && rank == r);
            const int src = __ffsll((long long)hit) - 1;
            // readlane moves 32 bits: the pointer goes over in two halves
            const uint64_t b = reinterpret_cast<uint64_t>(bp);
            const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, src);
            const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
            *blob_out = reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
            *p0_out = __builtin_amdgcn_readlane(o0, src);
            *p1_out = __builtin_amdgcn_readlane(o1, src);
            return e0 + src;
        }
        seen += n;
    }
    return -1;
}

// Marks a weight register as rewritten here, so that its unpacking is not
// hoisted above the point where the pipeline expects the load to have landed
// (a hoisted unpack waits for every load issued before it).
__device__ __forceinline__ void opaque(uint4_t &w) { asm volatile("" : "+v"(w)); }

// ROUTE: one token whose routing is still to be formed from the next-layer
// logit partials that the fused combine stored (DecodeRoute, moe_common.h).
// Every workgroup folds the partials in the pinned order, selects as the
// one-token router does and takes the blockIdx.y-th selected expert in id
// order (its sorted row); wave 0 of the first workgroup also writes the
// routing outputs, once its first weight loads are in flight.

constexpr int DECODE_XPRE = 4;   // up to this many tokens, all x rows are staged at entry
constexpr int DECODE_RG = 4;     // routed rows computed together from one weight unpack

// Memory behaviour the schedule is built around:
//  * the vector memory counter retires loads in issue order, so a value is
//    usable once it and every load issued before it have landed;
//  * a CU accepts only so many loads in flight: issuing the whole ~96 KB of
//    a workgroup up front stalls the issuing wave until most of it has come
//    back, and no arithmetic can run meanwhile.
// So each wave keeps PD weight chunks in flight and issues chunk i + PD just
// before it computes chunk i: the dot products run while later chunks
// stream.  Scales and activations go first (small).  Every weight address is
// in the global address space (a flat load would also count against the LDS
// counter and force a full drain at every LDS wait); no load is conditional.
// ZP: zero-point blobs (W = (u - z) s, z one byte per row and group in the
// scales' order); the correction constant of a chunk becomes per row:
// corr - z * sum (k_decode_frag.h).
template <int H, int G, int NW, int PD, bool ZP, bool ROUTE>
__global__ __launch_bounds__(NW * 64) void ffn_decode_kernel(
    const f16 *__restrict__ x, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, const uint8_t *const *__restrict__ blobs,
    const uint8_t *const *__restrict__ skip, int I, int E, int k, int ntk, int yflags,
    int64_t off_guq, int64_t off_dq, int64_t off_gus, int64_t off_ds, int64_t off_guz,
    int64_t off_dz, float *__restrict__ y, DecodeRoute rt)
{
    constexpr int NK = H / 32;                 // input chunks of gate/up rows
    constexpr int CPW = NK / NW;               // gate/up chunks per wave
    constexpr int NRB = H / 64;                // 64-row blocks of the down projection
    constexpr int RBW = NRB / NW;              // down blocks (chunks) per wave
    constexpr int NCH = CPW + RBW;             // weight chunks per wave
    constexpr int RG = DECODE_RG;
    constexpr int CPG = G / 32;                // chunks per scale group
    constexpr int NSG = CPW >= CPG ? CPW / CPG : 1;   // scale groups among a wave's chunks
    static_assert(NK % NW == 0 && NRB % NW == 0, "H/64 must be a multiple of the wave count");
    static_assert(NW >= RG, "one wave per row of a group does its SwiGLU");
    static_assert(DECODE_XPRE * CPW <= 64, "a wave stages its chunks of every token, a lane each");

    __shared__ __align__(16) half2_t xp[DECODE_XPRE][H / 2];   // prepared activations
    __shared__ float xc[DECODE_XPRE][NK];                     // their chunk constants
    __shared__ float xsum[ZP ? DECODE_XPRE : 1][ZP ? NK : 1];  // ZP: their chunk sums
    __shared__ float red[NW][RG][64];
    __shared__ __align__(16) half2_t hp[RG][16];              // prepared h chunks
    __shared__ int s_tok[RG];
    __shared__ float s_part[ROUTE ? 8 : 1][64];          // ROUTE: folded logit partials
    __shared__ uint64_t s_key[ROUTE ? NW : 1][64];      // ROUTE: each wave's selection keys
    __shared__ int s_cnt[ROUTE ? NW : 1][64];            // ROUTE: each wave's share of the ranks

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slice = blockIdx.x;
    const int T = ntk / k;
    const bool xpre = T <= DECODE_XPRE;
    // the blob section offsets are read now, while the expert lookup is in
    // flight, not after it (a late kernel-argument load would be waited for
    // at the first LDS wait)
    asm volatile("" ::"s"(off_guq), "s"(off_dq), "s"(off_gus), "s"(off_ds));
    if constexpr (ZP)
        asm volatile("" ::"s"(off_guz), "s"(off_dz));

    // activations of the whole (small) batch, each wave only the chunks it
    // multiplies: lane -> (token, chunk of the wave).  The loads go out now
    // and land during the expert lookup; each wave stages its own chunks, so
    // no workgroup barrier stands before the weight stream.
    // Unconditional loads (a lane without a chunk reads token 0's): no
    // branch around them, so the compiler's wait counts stay exact after it.
    half8_t xr[4];
    const bool xmine = xpre && lane < T * CPW;
    const int xt = lane / CPW, xcn = wave * CPW + lane % CPW;
    {
        const f16 *src = x + (size_t)(xmine ? xt : 0) * H + xcn * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xr[q] = ldg(reinterpret_cast<const half8_t *>(src + 8 * q));
    }

    const uint8_t *blob = nullptr;
    int p0 = 0, p1 = 0, route_rank = 0;
    float l_route = 0.0f;
    int e;
    if constexpr (ROUTE) {
        // The pinned fold of 64 partials is a butterfly (strides 32, 16, 8,
        // 4, 2, 1); after its first three levels, value r < 8 depends only on
        // partials r, r + 8, ..., r + 56.  So wave w loads those eight rows
        // for r = w (and w + 4 with four waves) and folds them in registers;
        // the eight values meet in LDS and every wave finishes the last
        // three levels.  The same additions as pinned_fold64.  Rows past nb
        // were never written and are zero.  The bias and the blob table are
        // requested at the same time.
        constexpr int NB = H / 8 < 64 ? H / 8 : 64;
        constexpr int CPV = 8 / NW;
        const bool ev = lane < E;
        float v[CPV][8];
#pragma unroll
        for (int q = 0; q < CPV; ++q)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int jj = wave + NW * q + 8 * m;
                v[q][m] = jj < NB ? ldg(rt.part + jj * 64 + lane) : 0.0f;
            }
        const float bv = rt.bias != nullptr && ev ? ldg(rt.bias + lane) : 0.0f;
        const uint8_t *bp = ev ? ldg(blobs + lane) : nullptr;
#pragma unroll
        for (int q = 0; q < CPV; ++q) {
            // v[q][m] is partial r + 8 m, r = wave + NW q
            const float a0 = v[q][0] + v[q][4], a1 = v[q][1] + v[q][5];   // stride 32
            const float a2 = v[q][2] + v[q][6], a3 = v[q][3] + v[q][7];
            const float b0 = a0 + a2, b1 = a1 + a3;                      // stride 16
            s_part[wave + NW * q][lane] = b0 + b1;                       // stride 8
        }
        __syncthreads();
        float c[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            c[r] = s_part[r][lane];
        const float d0 = c[0] + c[4], d1 = c[1] + c[5], d2 = c[2] + c[6], d3 = c[3] + c[7];
        const float e0 = d0 + d2, e1 = d1 + d3;
        float l = e0 + e1;
        if (rt.bias != nullptr)
            l = l + bv;
        // the one-token router's ranks: the number of keys that beat this
        // lane's.  Every wave holds all 64 keys; wave w counts only those of
        // lanes 64/NW w .. 64/NW (w + 1) - 1 (two waves share a SIMD, so 64
        // comparisons in every wave would be paid twice over), and the
        // counts meet in LDS.
        constexpr int KPW = 64 / NW;
        const uint64_t key = ev ? topk_key(l, lane) : 0ull;
        s_key[wave][lane] = key;
        __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
        int r0c = 0, r1c = 0;
#pragma unroll
        for (int jj = 0; jj < KPW; jj += 2) {
            const uint4_t q = *reinterpret_cast<const uint4_t *>(&s_key[wave][KPW * wave + jj]);
            r0c += (((uint64_t)q.y << 32) | q.x) > key ? 1 : 0;
            r1c += (((uint64_t)q.w << 32) | q.z) > key ? 1 : 0;
        }
        s_cnt[wave][lane] = r0c + r1c;
        __syncthreads();
        int rank = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            rank += s_cnt[w][lane];
        const bool sel = ev && rank < k;
        const uint64_t smask = __ballot(sel);
        const int a = blockIdx.y;
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const uint64_t hit = __ballot(sel && __popcll(smask & below) == a);
        e = hit ? __ffsll((long long)hit) - 1 : -1;   // the same in every wave
        if (e >= 0) {
            const uint64_t b = reinterpret_cast<uint64_t>(bp);
            const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, e);
            const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), e);
            blob = reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
            route_rank = __builtin_amdgcn_readlane(rank, e);
            p0 = a;
            p1 = a + 1;
        }
        l_route = l;
    } else {
        e = nth_active_expert(offsets, blobs, E, blockIdx.y, lane, &blob, &p0, &p1);
    }
    // an expert without weights in the table, or one that `skip` lists (done
    // by an earlier launch), is left to another launch
    if (e >= 0 && (blob == nullptr || (skip != nullptr && ldg(skip + e) != nullptr)))
        e = -1;
    if (e < 0)
        return;   // uniform over the workgroup: every wave found the same expert
    const int IC = I / 32;                     // input chunks of the down rows
    constexpr int HG = H / G;
    const int IG = I / G;
    const int nrows = p1 - p0;

    // flat indices t*k + j of the expert's first 64 rows (decode: at most 4
    // rows); needed for the token of a row (T > 1) and for a token-order y
    const bool tok_order = (yflags & YF_TOKEN_ORDER) != 0;
    const int prow = ROUTE ? (lane == 0 ? route_rank : 0)
                           : ((T > 1 || tok_order) && lane < nrows) ? ldg(perm + p0 + lane) : 0;

    // scales: one per scale group among this wave's gate/up chunks, one per
    // down block (2 bytes per lane each)
    const uint16_t *gus = reinterpret_cast<const uint16_t *>(blob + off_gus) +
                          (size_t)slice * HG * 64 + lane;
    uint16_t sgu[NSG];
#pragma unroll
    for (int j = 0; j < NSG; ++j)
        sgu[j] = ldg_nt(gus + (size_t)(((wave * CPW + j * CPG) * 32) / G) * 64);
    const uint16_t *dsc = reinterpret_cast<const uint16_t *>(blob + off_ds);
    uint16_t sd[RBW];
#pragma unroll
    for (int r = 0; r < RBW; ++r)
        sd[r] = ldg_nt(dsc + ((size_t)(wave * RBW + r) * IG + (slice * 32) / G) * 64 + lane);
    // zero points, in the scales' order (one byte each)
    uint8_t zgu[ZP ? NSG : 1], zd[ZP ? RBW : 1];
    if constexpr (ZP) {
        const uint8_t *guz = blob + off_guz + (size_t)slice * HG * 64 + lane;
#pragma unroll
        for (int j = 0; j < NSG; ++j)
            zgu[j] = ldg_nt(guz + (size_t)(((wave * CPW + j * CPG) * 32) / G) * 64);
        const uint8_t *dz = blob + off_dz;
#pragma unroll
        for (int r = 0; r < RBW; ++r)
            zd[r] = ldg_nt(dz + ((size_t)(wave * RBW + r) * IG + (slice * 32) / G) * 64 + lane);
    }

    // weight chunks of this wave: gate/up chunks 0..CPW-1 (one 1 KB run of the
    // fused 64-row block each), then its down blocks (the slice's 16-byte
    // column of 64 down rows each)
    const uint4_t *guq = reinterpret_cast<const uint4_t *>(blob + off_guq) +
                         ((size_t)slice * NK + (size_t)wave * CPW) * 64 + lane;
    const uint4_t *dqw = reinterpret_cast<const uint4_t *>(blob + off_dq) +
                         ((size_t)wave * RBW * IC + slice) * 64 + lane;
    uint4_t w[NCH];
    auto issue = [&](int i) {
        if (i < CPW)
            w[i] = ldg_nt(guq + (size_t)i * 64);
        else if (i < NCH)
            w[i] = ldg_nt(dqw + (size_t)(i - CPW) * IC * 64);
    };
#pragma unroll
    for (int i = 0; i < PD && i < NCH; ++i)
        issue(i);
    // ROUTE: the routing outputs, by one wave while the first weight chunks
    // are on their way (before them, they would delay this workgroup's
    // stream and so the whole launch)
    if constexpr (ROUTE) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && wave == 0)
            one_token_select(l_route, E, k, rt.flags, s_key[0], rt.idx, rt.w, rt.counts,
                             rt.offsets, rt.perm, rt.inv_perm, lane);
    }

    // pinned here: prepared any earlier, the wait for x would come before
    // the expert lookup is even issued
#pragma unroll
    for (int q = 0; q < 4; ++q)
        asm volatile("" : "+v"(xr[q]));
    if (xmine)
        prep_chunk_regs<ZP>(xr, &xp[xt][xcn * 16], &xc[xt][xcn], &xsum[ZP ? xt : 0][ZP ? xcn : 0]);

    // One group of R routed rows (R a constant, so that no register is held
    // for absent rows).  FIRST: the weights are still streaming in and the
    // group issues the rest of them as it goes.
    auto group = [&](auto first, auto rows, int r0) {
        constexpr bool FIRST = decltype(first)::value;
        constexpr int R = decltype(rows)::value;
        if (!xpre) {
            // stage this group's rows in slots 0..R-1
            if ((int)threadIdx.x < R)
                s_tok[threadIdx.x] = ldg(perm + p0 + r0 + threadIdx.x) / k;
            __syncthreads();
            for (int i = threadIdx.x; i < R * NK; i += NW * 64) {
                const int r = i / NK, c = i % NK;
                prep_chunk<ZP>(x + (size_t)s_tok[r] * H + c * 32, &xp[r][c * 16], &xc[r][c],
                               &xsum[ZP ? r : 0][ZP ? c : 0]);
            }
            lds_barrier();
        } else {
            wave_lds_sync();   // this wave's own staged chunks
        }
        // activation slot of each row: the token (all tokens staged), or the
        // row's place in the group; read after the barrier, so that the
        // token-id load never delays it
        int slot[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = r0 + r;
            if (!xpre)
                slot[r] = r;
            else if (T == 1)
                slot[r] = 0;
            else
                slot[r] = ((rr < 64) ? __shfl(prow, rr, 64) : ldg(perm + p0 + rr)) / k;
        }

        // gate/up rows (lane = row of the fused block), K split over waves
        float acc[R] = {};
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            if constexpr (FIRST)
                issue(i + PD);
            opaque(w[i]);
            half2_t m[16];
            unpack_chunk(w[i], m);
            const int c = wave * CPW + i;
            const float s = h2f(sgu[CPW >= CPG ? i / CPG : 0]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float c0 = xc[slot[r]][c];
                if constexpr (ZP)
                    c0 = fmaf(-(float)zgu[CPW >= CPG ? i / CPG : 0], xsum[slot[r]][c], c0);
                acc[r] = fmaf(dot_unpacked(m, &xp[slot[r]][c * 16], c0), s, acc[r]);
            }
        }
        if constexpr (FIRST) {
#pragma unroll
            for (int i = CPW + PD; i < NCH; ++i)
                issue(i);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            red[wave][r][lane] = acc[r];
        // unpack the down chunks while the other waves finish their gate/up
        // (up to two rows; with more, the registers of the unpacked chunks
        // are not there and each chunk is unpacked where it is used)
        constexpr bool PRE = R <= 2;
        half2_t md[PRE ? RBW : 1][16];
        if constexpr (PRE) {
#pragma unroll
            for (int j = 0; j < RBW; ++j) {
                opaque(w[CPW + j]);
                unpack_chunk(w[CPW + j], md[j]);
#pragma unroll
                for (int q = 0; q < 16; ++q)   // materialised here, not sunk past the barrier
                    asm volatile("" : "+v"(md[j][q]));
            }
        }
        lds_barrier();
        if (wave < R) {
            // wave r: h of row r for intermediate index lane (lanes < 32), fp16
            const int r = wave;
            float v = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2)
                v += red[w2][r][lane];
            const float up = __shfl(v, (lane + 32) & 63, 64);
            const f16 hq = (f16)swiglu_fast(v, up);
            const bool odd = (lane >> 1) & 1;
            if (lane < 32)
                reinterpret_cast<f16 *>(hp[r])[lane] = odd ? hq * (f16)0.0625f : hq;
        }
        lds_barrier();

        // each row's correction constant (see k_decode_frag.h): -1032 per
        // low-field h, -72 per high-field h = -1152 per prepared (h/16) value.
        // ZP: -1024 per low-field h, -64 per high-field h (-1024 per prepared
        // value), and the plain sum of h for the per-row -z * sum term
        float hc[R], hs[ZP ? R : 1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            hc[r] = 0.0f;
            if constexpr (ZP) {
                hs[r] = 0.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    hc[r] = dot2(hp[r][j], half2_t{(f16)-1024.0f, (f16)-1024.0f}, hc[r]);
                    hs[r] = dot2(hp[r][j], (j & 1) ? half2_t{(f16)16.0f, (f16)16.0f}
                                                   : half2_t{(f16)1.0f, (f16)1.0f}, hs[r]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    hc[r] = dot2(hp[r][j], (j & 1) ? half2_t{(f16)-1152.0f, (f16)-1152.0f}
                                                   : half2_t{(f16)-1032.0f, (f16)-1032.0f},
                                 hc[r]);
            }
        }

        // down strip: lane = output row, the 32 prepared h values from LDS
        // y row of each row of the group: its sorted position, or t*k + j
        // (pinned here: hoisted above the gate/up loop, the wait for the
        // token-id load would hold the first dot product)
        int pr = prow;
        asm volatile("" : "+v"(pr));
        int yrow[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = r0 + r;
            if (tok_order)   // uniform: every lane takes the same branch
                yrow[r] = (rr < 64) ? __shfl(pr, rr, 64) : ldg(perm + p0 + rr);
            else
                yrow[r] = p0 + rr;
        }
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
            const int rb = wave * RBW + j;
            const float s = h2f(sd[j]);
            half2_t mj[16];
            if constexpr (!PRE) {
                opaque(w[CPW + j]);
                unpack_chunk(w[CPW + j], mj);
            }
            // column rb * 64 + lane, stored at its partial-major position
            // when asked (a uniform choice)
            const int col = rb * 64 + lane;
            const int ycol = (yflags & YF_PARTIAL_ORDER) ? pm_col(col, H) : col;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float c0 = hc[r];
                if constexpr (ZP)
                    c0 = fmaf(-(float)zd[j], hs[r], c0);
                y[((size_t)slice * ntk + yrow[r]) * H + ycol] =
                        dot_unpacked(PRE ? md[j] : mj, hp[r], c0) * s;
            }
        }
    };

    using std::integral_constant;
    using std::true_type;
    const int R0 = min(RG, nrows);
    switch (R0) {
    case 1: group(true_type{}, integral_constant<int, 1>{}, 0); break;
    case 2: group(true_type{}, integral_constant<int, 2>{}, 0); break;
    case 3: group(true_type{}, integral_constant<int, 3>{}, 0); break;
    default: group(true_type{}, integral_constant<int, 4>{}, 0); break;
    }
    // more rows than a group (only with more than DECODE_XPRE tokens): one
    // row at a time from the weights now in registers
    for (int r0 = R0; r0 < nrows; ++r0) {
        lds_barrier();   // the previous group is done with xp, red and hp
        group(std::false_type{}, integral_constant<int, 1>{}, r0);
    }
}

constexpr int DECODE_PD = 4;   // weight chunks each wave keeps in flight

template <int H, bool ZP, bool ROUTE>
static int launch_decode_h(dim3 grid, hipStream_t s, const f16 *x, const int32_t *perm,
                           const int32_t *offsets, const uint8_t *const *blobs,
                           const uint8_t *const *skip, int I, int E, int k, int g, int ntk,
                           int yflags, const DevLayout &L, float *y, const DecodeRoute &rt)
{
    constexpr int NW = (H >= 1024) ? 8 : 4;
#define MOE_DECODE_LAUNCH(G)                                                                  \
    hipLaunchKernelGGL((ffn_decode_kernel<H, G, NW, DECODE_PD, ZP, ROUTE>), grid,              \
                       dim3(NW * 64), 0, s, x, perm, offsets, blobs, skip, I, E, k, ntk, yflags, \
                       L.gu_q, L.d_q, L.gu_s, L.d_s, L.gu_z, L.d_z, y, rt)
    switch (g) {
    case 32: MOE_DECODE_LAUNCH(32); break;
    case 64: MOE_DECODE_LAUNCH(64); break;
    case 128: MOE_DECODE_LAUNCH(128); break;
    default: return set_error(MOE_EUNSUPPORTED, "decode kernel: group %d not instantiated", g);
    }
#undef MOE_DECODE_LAUNCH
    return MOE_OK;
}

// skip (may be null): a device table of E pointers; experts with a non-null
// entry there are not computed (an earlier launch did them).  Experts with a
// null entry in `blobs` are not computed either.  rt (may be null): route one
// token (E <= 64) from logit partials first (perm and offsets unused; the
// caller has checked the shape).
int launch_ffn_decode(const void *x, const int32_t *perm, const int32_t *offsets,
                      const void *const *blobs, const void *const *skip, int T, int H, int I,
                      int E, int k, int g, int fmt, int yflags, float *y, hipStream_t s,
                      const DecodeRoute *rt)
{
    const int ntk = T * k;
    if (ntk == 0)
        return MOE_OK;
    const DevLayout L = dev_layout(H, I, g, fmt);
    dim3 grid(I / 32, (unsigned)min(E, ntk));
    const f16 *xh = static_cast<const f16 *>(x);
    const uint8_t *const *b = reinterpret_cast<const uint8_t *const *>(blobs);
    const uint8_t *const *sk = reinterpret_cast<const uint8_t *const *>(skip);
    int rc;
    const DecodeRoute rr = rt ? *rt : DecodeRoute{};
#define MOE_DECODE_H2(HH, R)                                                                   \
    rc = fmt == FMT_ZP                                                                         \
             ? launch_decode_h<HH, true, R>(grid, s, xh, perm, offsets, b, sk, I, E, k, g, ntk, \
                                            yflags, L, y, rr)                                  \
             : launch_decode_h<HH, false, R>(grid, s, xh, perm, offsets, b, sk, I, E, k, g,    \
                                             ntk, yflags, L, y, rr)
#define MOE_DECODE_H(HH)                                                                       \
    if (rt) {                                                                                  \
        MOE_DECODE_H2(HH, true);                                                               \
    } else {                                                                                   \
        MOE_DECODE_H2(HH, false);                                                              \
    }
    switch (H) {
    case 256: MOE_DECODE_H(256) break;
    case 512: MOE_DECODE_H(512) break;
    case 1024: MOE_DECODE_H(1024) break;
    case 2048: MOE_DECODE_H(2048) break;
    default: return set_error(MOE_EUNSUPPORTED, "decode kernel: H=%d not instantiated", H);
    }
#undef MOE_DECODE_H
#undef MOE_DECODE_H2
    if (rc != MOE_OK)
        return rc;
    MOE_LAUNCH_CHECK("ffn_decode_kernel");
    return MOE_OK;
}

}  // namespace moe
