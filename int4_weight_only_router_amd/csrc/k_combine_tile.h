// k_combine_tile.h -- one block's share of the router-weighted combine of
// decode partials, shared by the combine kernel and the fused
// combine-and-route kernel so that both round identically.
//
// Horizon RunMap "03 / Arquitetura": the experts' results return to the rest
// of the model weighted by the router.  For token t and column c:
//   out = fp16_rne( sum_j w[t,j] * Y_j + s[t,c] + r[t,c] ),
//   Y_j = sum over slices of y[slice][inv_perm[t*k+j]][c],
// in fp32 in a fixed order: the slices in two contiguous halves, each in
// slice order, the halves then added; experts j ascending, then the shared
// term, then the residual.
#pragma once

#include "moe_common.h"

namespace moe {

typedef float float4_t __attribute__((ext_vector_type(4)));

// Shared-expert gate of one token formed by one wave: fp32 dot of x_t with wsg
// (8 columns per lane per pass), summed across the wave, then the sigmoid.
// Every lane returns the same value.
__device__ inline float shared_gate_wave(const f16 *__restrict__ xt, const f16 *__restrict__ wsg,
                                         int H, int lane)
{
    float a = 0.0f;
#pragma unroll 4
    for (int c = lane * 8; c < H; c += 64 * 8) {
        const half8_t xv = *reinterpret_cast<const half8_t *>(xt + c);
        const half8_t wv = *reinterpret_cast<const half8_t *>(wsg + c);
#pragma unroll
        for (int m = 0; m < 8; ++m)
            a = __builtin_fmaf((float)xv[m], (float)wv[m], a);
    }
    a = wave_sum_f32(a);
    return 1.0f / (1.0f + expf(-a));
}

// R runs of up to 32 columns of one token by a group of 256 threads (tid =
// index in the group) as 2 slice halves x 16 expert slots x 8 column quads;
// run r's i-th column is cols.col(r, i), found in y at cols.y(r, i); the four
// y positions of a quad are consecutive.  A block may hold several groups,
// each with its own R CombineTileSmem.
struct CombineTileSmem {
    float part[2][16][33];
    float gate;
};

struct ContigCols {   // one run: columns base .. base + 31, y in plain order
    int base;
    __device__ int col(int, int i) const { return base + i; }
    __device__ int y(int, int i) const { return base + i; }
};

// One run of y positions base .. base + 31 in partial-major order
// (MOE_DTYPE_F32_PM); the output column is the position's original column.
struct PmCols {
    int base, H;
    __device__ int col(int, int i) const
    {
        const int q = (H / 8 + 63) / 64;
        const int s = (base + i) >> 3;   // stored chunk j q + m
        return ((s % q) * 64 + s / q) * 8 + ((base + i) & 7);
    }
    __device__ int y(int, int i) const { return base + i; }
};

// Thread (g, j, q) sums 4 columns of expert slot j of every run over the g-th
// half of the S slices, in slice order, with 16-byte loads issued in batches
// of 16 per run; the first R * 32 threads (run r = tid / 32, column
// i = tid % 32 < ncols) then form Y_j = half_0 + half_1 and fold w[t,j] Y_j in
// j order, then the shared and residual terms, and return the fp16 result
// (also stored to out when out is given).  The finishing threads load their
// weights, shared and residual values before the slice loads, unconditionally
// (from a readable stand-in address when a term is absent), so no wait for
// them precedes the slice loads and nothing after the barrier waits on
// memory.  GATED: the group's last wave forms the gate from the layer input x
// after its own loads (with k <= 8 it has none).  Every thread of the block
// must call this (it holds a block-wide barrier).
template <bool GATED, int R, typename Cols>
__device__ __forceinline__ f16 combine_tile(const float *__restrict__ y, int S,
                                            const int32_t *__restrict__ inv_perm,
                                            const float *__restrict__ w,
                                            const float *__restrict__ shared,
                                            const f16 *__restrict__ x,
                                            const f16 *__restrict__ wsg, const f16 *residual,
                                            int T, int t, int H, int k, int ncols, Cols cols,
                                            f16 *out, CombineTileSmem *sm, int tid)
{
    constexpr int SB = 16;   // loads in flight per batch and run
    const int q = tid & 7;
    const int j = (tid >> 3) & 15;
    const int g = tid >> 7;
    const int fr = tid >> 5, fi = tid & 31;   // finishing thread: run, column
    const bool fin = fr < R && fi < ncols;
    const int cf = fin ? cols.col(fr, fi) : 0;
    float wj[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
        wj[jj] = w[(size_t)t * k + min(jj, k - 1)];
    const float *shp = shared ? shared + (size_t)t * H + cf : y;
    const f16 *rsp = residual ? residual + (size_t)t * H + cf : reinterpret_cast<const f16 *>(y);
    const float sh = *shp;
    const f16 rs = *rsp;

    const int half = (S + 1) / 2;
    const int sb = g * half, se = min(S, sb + half);
    if (j < k && 4 * q < ncols) {
        const size_t f = (size_t)t * k + j;
        const size_t p = inv_perm ? (size_t)inv_perm[f] : f;   // NULL: y in token order
        const size_t stride = (size_t)T * k * H;
        float4_t v[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            v[r] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = sb; s0 < se; s0 += SB) {
            float4_t vb[R][SB];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float *src = y + p * H + cols.y(r, 4 * q);
#pragma unroll
                for (int i = 0; i < SB; ++i)   // past se: slice se - 1 again, not added
                    vb[r][i] = *reinterpret_cast<const float4_t *>(
                        src + (size_t)min(s0 + i, se - 1) * stride);
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < SB; ++i)
                    if (s0 + i < se) {
                        v[r][0] += vb[r][i][0];
                        v[r][1] += vb[r][i][1];
                        v[r][2] += vb[r][i][2];
                        v[r][3] += vb[r][i][3];
                    }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                sm[r].part[g][j][q * 4 + m] = v[r][m];
    }
    if constexpr (GATED) {
        if (tid >= 192) {
            const float gv = shared_gate_wave(x + (size_t)t * H, wsg, H, tid & 63);
            if (tid == 192)
                sm[0].gate = gv;
        }
    }
    __syncthreads();
    f16 o = (f16)0.0f;
    if (fin) {
        const CombineTileSmem &m = sm[fr];
        float acc = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            if (jj < k) {
                const float yj = m.part[0][jj][fi] + m.part[1][jj][fi];
                acc = __builtin_fmaf(wj[jj], yj, acc);
            }
        }
        if (shared)
            acc += GATED ? sm[0].gate * sh : sh;
        if (residual)
            acc += (float)rs;
        o = (f16)acc;
        if (out)
            out[(size_t)t * H + cf] = o;
    }
    return o;
}

}  // namespace moe
