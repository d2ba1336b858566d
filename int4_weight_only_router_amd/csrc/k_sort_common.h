// k_sort_common.h -- device helpers shared by the permutation kernels.
#pragma once

#include "moe_common.h"

namespace moe {

// Stable scatter of flat elements [f0, f1) by one wave (f1 - f0 <= 64 *
// WS_GROUPS per call; callers loop).  cnt[e] holds the next free sorted
// position of expert e.  All keys of the range are loaded first (one memory
// round trip, not one per group).  Per group of 64 elements, a lane's peers
// (lanes holding the same key) come from one ballot per key bit; its rank is
// the number of peers in lower lanes, and the lowest peer advances cnt[key]
// by the group's multiplicity.  Out-of-range ids are skipped.
constexpr int WS_GROUPS = 8;

__device__ __forceinline__ void wave_scatter(const int32_t *__restrict__ idx, int f0, int f1,
                                             int E, int *cnt, int32_t *__restrict__ perm,
                                             int32_t *__restrict__ inv_perm, int lane)
{
    const int kbits = 32 - __builtin_clz((unsigned)max(E - 1, 1));
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base0 = f0; base0 < f1; base0 += 64 * WS_GROUPS) {
        int keys[WS_GROUPS];
#pragma unroll
        for (int g = 0; g < WS_GROUPS; ++g) {
            const int f = base0 + 64 * g + lane;
            keys[g] = (f < f1) ? idx[f] : -1;
        }
#pragma unroll
        for (int g = 0; g < WS_GROUPS; ++g) {
            const int f = base0 + 64 * g + lane;
            const int key = keys[g];
            const bool valid = (unsigned)key < (unsigned)E;
            uint64_t peers = __ballot(valid);
            if (peers == 0)
                continue;   // uniform: nothing left in this group
            for (int b = 0; b < kbits; ++b) {
                const bool bit = (key >> b) & 1;
                const uint64_t m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            const int rank = __popcll(peers & below);
            int pos = 0;
            if (valid)
                pos = cnt[key] + rank;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                if (rank == 0)
                    cnt[key] = pos + __popcll(peers);
                perm[pos] = f;
                inv_perm[f] = pos;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// Counts, offsets and running positions of n flat elements by one wave
// (histogram in LDS cnt[E], exclusive scan); afterwards cnt[e] = offsets[e].
__device__ __forceinline__ void wave_count_scan(const int32_t *__restrict__ idx, int n, int E,
                                                int *cnt, int32_t *__restrict__ counts,
                                                int32_t *__restrict__ offsets, int lane)
{
    for (int e = lane; e < E; e += 64)
        cnt[e] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int f0 = 0; f0 < n; f0 += 64 * WS_GROUPS) {   // keys loaded a batch at a time
        int keys[WS_GROUPS];
#pragma unroll
        for (int g = 0; g < WS_GROUPS; ++g) {
            const int f = f0 + 64 * g + lane;
            keys[g] = (f < n) ? idx[f] : -1;
        }
#pragma unroll
        for (int g = 0; g < WS_GROUPS; ++g)
            if ((unsigned)keys[g] < (unsigned)E)
                atomicAdd(&cnt[keys[g]], 1);
    }
    __builtin_amdgcn_wave_barrier();
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int seg = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E)
            seg += cnt[e0 + i];
    int incl = seg;
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
        int o = __shfl_up(incl, st, 64);
        if (lane >= st)
            incl += o;
    }
    int run = incl - seg;
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i < per; ++i) {
        int e = e0 + i;
        if (e < E) {
            int c = cnt[e];
            counts[e] = c;
            offsets[e] = run;
            cnt[e] = run;
            run += c;
        }
    }
    if (lane == 63)
        offsets[E] = run;
    __builtin_amdgcn_wave_barrier();
}

// The router's pinned cross-lane sum of 64 partials: a_j += a_(j xor off)
// for off = 32, 16, 8, 4, 2, 1 in that order, every lane ending with the
// same value.  Each step adds exactly the value of lane j xor off, fetched
// with the cheapest exchange that gives it: a permute across the two
// halves (32), a swizzle inside each 32 lanes (16), and register moves
// inside each 16-lane row -- rotate by 8 (8); shift left / right by 4, each
// lane taking the side that lands on j xor 4 (4); quad permutes (2, 1).
// Bit-identical to six __shfl_xor steps; all 64 lanes must be active.
__device__ __forceinline__ float pinned_xor_sum(float a, int lane)
{
    a = a + __shfl_xor(a, 32, 64);
    a = a + __builtin_bit_cast(float,
                               __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, a), 0x401F));
    a = a + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                  0x128, 0xF, 0xF, false));
    const int ai = __builtin_bit_cast(int, a);
    const int up = __builtin_amdgcn_update_dpp(0, ai, 0x104, 0xF, 0xF, false);   // from j + 4
    const int dn = __builtin_amdgcn_update_dpp(0, ai, 0x114, 0xF, 0xF, false);   // from j - 4
    a = a + __builtin_bit_cast(float, (lane & 4) ? dn : up);
    a = a + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                  0x4E, 0xF, 0xF, false));
    a = a + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a),
                                                                  0xB1, 0xF, 0xF, false));
    return a;
}

// The same butterfly with all 64 partials held by one lane: after the step
// of stride `off`, partial j (j < off) holds p_j + p_(j+off), exactly what
// lane j (and lane j xor off) holds after that step of pinned_xor_sum, so
// the result has the same bits.
__device__ __forceinline__ float pinned_fold64(float (&p)[64])
{
#pragma unroll
    for (int off = 32; off; off >>= 1) {
#pragma unroll
        for (int j = 0; j < off; ++j)
            p[j] = p[j] + p[j + off];
    }
    return p[0];
}

struct Cand {
    float v;
    int e;   // -1: empty slot
};

// Selection key: a strictly larger key ranks before in the selection order
// (logit descending, then lower expert index), as one unsigned 64-bit compare.  High word: the logit's bits made monotonic
// (negative values inverted, positive ones offset by the sign bit; -0 is
// first turned into +0 so that equal logits tie); low word: 0xFFFF - e, so
// that on a tie the lower expert index ranks first.  Empty slots use key 0,
// below every finite logit.
__device__ __forceinline__ uint64_t topk_key(float v, int e)
{
    const int u = __builtin_bit_cast(int, v + 0.0f);
    const uint32_t o = (uint32_t)(u ^ ((u >> 31) | (int)0x80000000));
    return ((uint64_t)o << 32) | (uint32_t)(0xFFFF - e);
}

// Selection, softmax and sort of one token over at most 64 experts by one
// wave, lane e holding expert e's logit l (ignored for e >= E); `bkey` is 64
// keys of LDS.  Ranks come from counting the keys that beat each lane's key;
// the softmax maximum is the logit ranked first; the denominators use the
// fixed-order wave sum.  Writes the k selected (idx, weight) pairs in rank
// order and the stable sort of one token's k distinct experts: counts 0/1,
// offsets = selected experts of lower id (offsets[E] = k), perm[off] = rank,
// inv_perm[rank] = off.  With a host mirror (HostMirror) the selected ids
// are also written there, then the mirror's flag.
__device__ __forceinline__ void one_token_select(float l, int E, int k, unsigned flags,
                                                 uint64_t *bkey, int32_t *__restrict__ idx_out,
                                                 float *__restrict__ w_out,
                                                 int32_t *__restrict__ counts,
                                                 int32_t *__restrict__ offsets,
                                                 int32_t *__restrict__ perm,
                                                 int32_t *__restrict__ inv_perm, int lane,
                                                 HostMirror hm = HostMirror{nullptr, nullptr, 0u})
{
    const int e = lane;
    const bool valid = e < E;
    const uint64_t key = valid ? topk_key(l, e) : 0ull;
    bkey[lane] = key;
    __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
        const uint4_t q = *reinterpret_cast<const uint4_t *>(bkey + j);
        const uint4_t p = *reinterpret_cast<const uint4_t *>(bkey + j + 2);
        r0 += (((uint64_t)q.y << 32) | q.x) > key ? 1 : 0;
        r1 += (((uint64_t)q.w << 32) | q.z) > key ? 1 : 0;
        r2 += (((uint64_t)p.y << 32) | p.x) > key ? 1 : 0;
        r3 += (((uint64_t)p.w << 32) | p.z) > key ? 1 : 0;
    }
    const int rank = (r0 + r1) + (r2 + r3);
    const bool sel = valid && rank < k;
    // softmax over all E: the maximum is the logit ranked first
    const int top = __ffsll((long long)__ballot(valid && rank == 0)) - 1;
    const float m =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), top));
    const float pe = valid ? expf(l - m) : 0.0f;
    const float den = wave_sum_f32(pe);   // softmax denominator (order fixed, not pinned)
    float p = pe / den;
    if (flags & MOE_RENORM) {
        const float ws = wave_sum_f32(sel ? p : 0.0f);
        p = p / ws;
    }
    if (sel) {
        idx_out[rank] = e;
        w_out[rank] = p;
        if (hm.ids)
            __hip_atomic_store(hm.ids + rank, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (hm.ids) {
        // the fence's wait covers the id stores of every lane of this wave
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
        if (lane == 0)
            __hip_atomic_store(hm.flag, hm.seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // position = selected experts of lower id, flat index = rank
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int off = __popcll(__ballot(sel) & below);
    if (valid) {
        counts[e] = sel ? 1 : 0;
        offsets[e] = off;
    }
    if (lane == E - 1)
        offsets[E] = k;
    if (sel) {
        perm[off] = rank;
        inv_perm[rank] = off;
    }
}

// One step of a wave-wide maximum of 64-bit keys: each lane takes the larger
// of its key and that of the lane DPP pattern CTRL names (a permutation
// inside each 16-lane row, so every source lane exists).  Register moves
// only: no LDS round trip per step.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t a)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)a, CTRL, 0xF, 0xF,
                                                              false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(a >> 32), CTRL,
                                                              0xF, 0xF, false);
    const uint64_t b = ((uint64_t)hi << 32) | lo;
    return b > a ? b : a;
}

// Maximum of one key per lane over the wave, returned to every lane: within
// each row by quad swaps (xor 1, xor 2), the half-row mirror and the row
// mirror, then across the four rows by reading lanes 0, 16, 32 and 48.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t a)
{
    a = dpp_max_step<0xB1>(a);    // quad_perm [1,0,3,2]
    a = dpp_max_step<0x4E>(a);    // quad_perm [2,3,0,1]
    a = dpp_max_step<0x141>(a);   // row_half_mirror: 8-lane halves
    a = dpp_max_step<0x140>(a);   // row_mirror: 16-lane rows
    uint64_t m = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)a, 16 * r);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), 16 * r);
        const uint64_t v = ((uint64_t)hi << 32) | lo;
        m = v > m ? v : m;
    }
    return m;
}

// Top-k of one token's E logits by one wave (E <= 64*NV): lane l holds the
// selection keys of experts l, l+64, ...; k rounds, each taking the largest
// remaining key (a per-lane scan, then wave_max_u64, so every lane agrees)
// and clearing it at its owner lane.  The key orders exactly as the
// selection order (logit desc, index asc); the logit is recovered from the
// key's high word.  sel[0..k) receives the pairs in order.
template <int NV>
__device__ __forceinline__ void wave_topk_nv(const float *l, int E, int k, int lane, Cand *sel)
{
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? topk_key(l[e], e) : 0ull;
    }
    for (int j = 0; j < k; ++j) {
        uint64_t b = key[0];
#pragma unroll
        for (int i = 1; i < NV; ++i)
            b = key[i] > b ? key[i] : b;
        b = wave_max_u64(b);
        const int e = 0xFFFF - (int)(uint32_t)(b & 0xFFFFu);
        const uint32_t o = (uint32_t)(b >> 32);
        const uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
        if (lane == 0)
            sel[j] = Cand{__builtin_bit_cast(float, u), e};
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (e == lane + 64 * i)
                key[i] = 0ull;
    }
}

// LDS scratch of one wave_topk call: the blocks' candidates (nb*16), their
// keys, and the 64 keys of the block being ranked (16-byte aligned; the size
// is a multiple of 16).
__host__ __device__ constexpr size_t topk_scratch_bytes(int E)
{
    return (size_t)((E + 63) / 64) * 16 * (sizeof(Cand) + sizeof(uint64_t)) + 64 * sizeof(uint64_t);
}

// Local top-k of one block of 64 experts of a token, by one wave: lane i
// holds expert 64b+i and writes its key to bkey[i]; its rank inside the
// block is the number of larger keys (broadcast 16-byte reads, one 64-bit
// compare and one add per key), and ranks below k land in cand/ckey[0..k).
// Slots past the block's size are empty (e = -1, key 0).
__device__ __forceinline__ void block_topk(const float *l, int E, int k, int b, int lane,
                                           Cand *cand, uint64_t *ckey, uint64_t *bkey)
{
    const int e0 = 64 * b;
    const int e = e0 + lane;
    const bool valid = e < E;
    const float v = valid ? l[e] : 0.0f;
    const uint64_t key = valid ? topk_key(v, e) : 0ull;
    bkey[lane] = key;
    __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
    // four independent counts, so the compares do not form one serial chain
    int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
        const uint4_t q = *reinterpret_cast<const uint4_t *>(bkey + j);
        const uint4_t p = *reinterpret_cast<const uint4_t *>(bkey + j + 2);
        r0 += (((uint64_t)q.y << 32) | q.x) > key ? 1 : 0;
        r1 += (((uint64_t)q.w << 32) | q.z) > key ? 1 : 0;
        r2 += (((uint64_t)p.y << 32) | p.x) > key ? 1 : 0;
        r3 += (((uint64_t)p.w << 32) | p.z) > key ? 1 : 0;
    }
    const int rank = (r0 + r1) + (r2 + r3);
    __builtin_amdgcn_wave_barrier();   // bkey is reused by the next block
    if (valid && rank < k) {
        cand[rank] = Cand{v, e};
        ckey[rank] = key;
    }
    if (!valid && lane < k) {   // fewer than k members: the remaining slots are empty
        cand[lane] = Cand{0.0f, -1};
        ckey[lane] = 0ull;
    }
}

// Global top-k of one token from its C block candidates (keys in ckey), by
// one wave.  Writes the chosen (logit, expert) in order to sel[0..k).
__device__ __forceinline__ void merge_topk(const Cand *cand, const uint64_t *ckey, int C, int k,
                                           int lane, Cand *sel)
{
    for (int c = lane; c < C; c += 64) {
        const uint64_t me = ckey[c];
        int rank = 0;
        int j = 0;
        for (; j + 2 <= C; j += 2) {   // ckey is 16-byte aligned
            const uint4_t q = *reinterpret_cast<const uint4_t *>(ckey + j);
            rank += (((uint64_t)q.y << 32) | q.x) > me ? 1 : 0;
            rank += (((uint64_t)q.w << 32) | q.z) > me ? 1 : 0;
        }
        if (j < C)
            rank += ckey[j] > me ? 1 : 0;
        if (me != 0ull && rank < k)
            sel[rank] = cand[c];
    }
}

// Top-k of one token's E logits (E <= 64 * NVMAX, NVMAX <= 16) by one wave
// into sel[0..k).  Up to two 64-expert blocks: rank-based (no dependent
// cross-lane chain); above: k argmax rounds.  scratch: topk_scratch_bytes(E)
// bytes of LDS, 16-byte aligned.  A kernel that only ever sees E <= 128
// instantiates it with NVMAX = 2 and carries none of the argmax variants.
// Blocks up to which the rank-based selection is used; with more, k argmax
// rounds are faster (measured at 512 experts: 14.3 against 19.3 us for the
// whole one-token route+sort launch).
constexpr int TOPK_RANK_MAX_NB = 2;

template <int NVMAX>
__device__ __forceinline__ void wave_topk_t(const float *l, int E, int k, int lane, Cand *sel,
                                            unsigned char *scratch)
{
    const int nb = (E + 63) >> 6;
    if (NVMAX <= 2 || nb <= TOPK_RANK_MAX_NB) {
        Cand *cand = reinterpret_cast<Cand *>(scratch);
        uint64_t *ckey = reinterpret_cast<uint64_t *>(cand + nb * 16);
        uint64_t *bkey = ckey + nb * 16;
        if (nb == 1) {
            // one block: its ranks are the final ones (k <= E fills every slot)
            block_topk(l, E, k, 0, lane, sel, ckey, bkey);
        } else {
            for (int b = 0; b < nb; ++b)
                block_topk(l, E, k, b, lane, cand + b * k, ckey + b * k, bkey);
            __builtin_amdgcn_wave_barrier();
            merge_topk(cand, ckey, nb * k, k, lane, sel);
        }
    } else if constexpr (NVMAX > 2) {
        if (NVMAX <= 4 || nb <= 4)
            wave_topk_nv<4>(l, E, k, lane, sel);
        else if constexpr (NVMAX > 4) {
            if (NVMAX <= 8 || nb <= 8)
                wave_topk_nv<8>(l, E, k, lane, sel);
            else
                wave_topk_nv<16>(l, E, k, lane, sel);
        }
    }
}

__device__ __forceinline__ void wave_topk(const float *l, int E, int k, int lane, Cand *sel,
                                          unsigned char *scratch)
{
    wave_topk_t<16>(l, E, k, lane, sel, scratch);
}

// Stable sorted position of each of n keys (flat order f) by one wave:
// pos(f) = #{g : key_g < key_f} + #{g < f : key_g == key_f}.
__device__ __forceinline__ void wave_stable_positions(const int *keys, int n, int32_t *perm,
                                                      int32_t *inv_perm, int lane)
{
    for (int f = lane; f < n; f += 64) {
        const int key = keys[f];
        int pos = 0;
        for (int g = 0; g < n; ++g) {
            const int kg = keys[g];
            pos += (kg < key || (kg == key && g < f)) ? 1 : 0;
        }
        perm[pos] = f;
        inv_perm[f] = pos;
    }
}

// Counting sort of n small keys (n <= 128) by one wave, without atomics:
// counts[e] = #{g : key_g == e}, offsets[e] = #{g : key_g < e}, positions as
// in wave_stable_positions.
__device__ __forceinline__ void wave_small_sort(const int *keys, int n, int E,
                                                int32_t *counts, int32_t *offsets,
                                                int32_t *perm, int32_t *inv_perm, int lane)
{
    for (int e = lane; e < E; e += 64) {
        int lt = 0, eq = 0;
        for (int g = 0; g < n; ++g) {
            const int kg = keys[g];
            lt += kg < e ? 1 : 0;
            eq += kg == e ? 1 : 0;
        }
        offsets[e] = lt;
        counts[e] = eq;
    }
    if (lane == 0)
        offsets[E] = n;
    wave_stable_positions(keys, n, perm, inv_perm, lane);
}

}  // namespace moe
