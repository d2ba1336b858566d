// k_decode_frag.h -- the decode GEMV's dot product on undecoded INT4
// nibbles and its activation preparation, shared by the decode kernels.
#pragma once

#include "moe_common.h"

namespace moe {

// The dot products take the weights as "magic" fp16 values without decoding
// them: OR-ing a nibble into the mantissa of 1024.0 gives v = 1024 + u (low
// field of a half, bits 0..3) or v = 1024 + 16u (high field, bits 4..7).  With
// the activation pair of a high field pre-divided by 16 (exact: a power of
// two), v * x' = 1024 x + u x or 64 x + u x, and the chunk sum of
// (u - 8) x = q x follows by starting the accumulator at
// -1032 * (sum of x over low-field pairs) - 72 * (sum over high-field pairs).
// That constant depends only on the activations, so it is computed once per
// token and chunk.  Pair p of a 32-element chunk is a high-field pair iff p is
// odd (device nibble layout).  The fp32 running sums stay within a few
// thousand, so rounding is ~1e-7 relative to them: far inside the budget.
// The 16 magic-value pairs of one chunk word, in activation-pair order.
__device__ __forceinline__ void unpack_chunk(uint4_t w, half2_t (&m)[16])
{
    const uint32_t M = 0x64006400u;
    // device chunk words hold elements 0-7, 16-23, 8-15, 24-31 in that order
    const uint32_t ws[4] = {w.x, w.z, w.y, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t v = ws[j], v8 = ws[j] >> 8;
        m[4 * j + 0] = __builtin_bit_cast(half2_t, (v & 0x000F000Fu) | M);
        m[4 * j + 1] = __builtin_bit_cast(half2_t, (v & 0x00F000F0u) | M);
        m[4 * j + 2] = __builtin_bit_cast(half2_t, (v8 & 0x000F000Fu) | M);
        m[4 * j + 3] = __builtin_bit_cast(half2_t, (v8 & 0x00F000F0u) | M);
    }
}

// d + the chunk's dot product from unpacked magic values and prepared
// activations (d starts at the chunk's correction constant).
__device__ __forceinline__ float dot_unpacked(const half2_t (&m)[16], const half2_t *xp, float d)
{
#pragma unroll
    for (int j = 0; j < 16; ++j)
        d = dot2(m[j], xp[j], d);
    return d;
}

// Prepares one 32-element chunk of activations (already in registers):
// pairs with odd index divided by 16, and the chunk's correction constant.
// Symmetric codes (z = 8): corr = -1032 * (low-field sum) - 72 * (high-field
// sum).  With a zero point z per group the constant is corr - z * sum, so the
// zero-point format keeps corr = -1024 * low - 64 * high and the plain sum
// (*sum) for the per-row term.
template <bool ZP = false>
__device__ __forceinline__ void prep_chunk_regs(const half8_t (&xv)[4], half2_t *dst, float *corr,
                                                float *sum = nullptr)
{
    float slo = 0.0f, shi = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const half8_t v = xv[q];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f16 a = v[2 * m], b = v[2 * m + 1];
            if (m & 1) {
                shi += (float)a + (float)b;
                dst[4 * q + m] = half2_t{a * (f16)0.0625f, b * (f16)0.0625f};
            } else {
                slo += (float)a + (float)b;
                dst[4 * q + m] = half2_t{a, b};
            }
        }
    }
    if constexpr (ZP) {
        *corr = -1024.0f * slo - 64.0f * shi;
        *sum = slo + shi;
    } else {
        *corr = -1032.0f * slo - 72.0f * shi;
    }
}

// The same, loading the chunk from memory first.
template <bool ZP = false>
__device__ __forceinline__ void prep_chunk(const f16 *src, half2_t *dst, float *corr,
                                           float *sum = nullptr)
{
    half8_t xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        xv[q] = *reinterpret_cast<const half8_t *>(src + 8 * q);
    prep_chunk_regs<ZP>(xv, dst, corr, sum);
}

}  // namespace moe
