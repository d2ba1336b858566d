// k_w4_frag.h -- MFMA operand helpers shared by the INT4 expert GEMMs:
// weight-word dequantisation into fp16 B fragments, global-address-space
// loads and the SwiGLU epilogue.
#pragma once

#include "moe_common.h"

namespace moe {

typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));

// One dword of 8 nibbles (device order) times its group scale -> the 8 fp16
// B-operand values of one lane for one 16-K step, fp16(q * s) exactly.  OR-ing
// a nibble into the mantissa of 1024.0 gives 1024 + u (bits 0..3 of a half)
// or 1024 + 16u (bits 4..7); subtracting 1032, or scaling by 1/16 and
// subtracting 72, gives q = u - 8 exactly.  `magic` holds 0x64006400 in a
// register so that mask-and-insert is one v_and_or_b32.
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s2, uint32_t magic)
{
    const uint32_t w8 = w >> 8;
    const half2_t k1032 = {(f16)-1032.0f, (f16)-1032.0f};
    const half2_t s16 = {(f16)0.0625f, (f16)0.0625f};
    const half2_t k72 = {(f16)-72.0f, (f16)-72.0f};
    half2_t q[4];
    q[0] = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) | magic) + k1032;
    q[1] = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) | magic) * s16 + k72;
    q[2] = __builtin_bit_cast(half2_t, (w8 & 0x000F000Fu) | magic) + k1032;
    q[3] = __builtin_bit_cast(half2_t, (w8 & 0x00F000F0u) | magic) * s16 + k72;
    half8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t v = q[i] * s2;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

// Zero-point codes: the same conversion with the offsets of the row's group,
// klo = -(1024 + z) and khi = -(64 + z) (both exact in fp16), giving
// fp16((u - z) * s) with one rounding.
__device__ __forceinline__ half8_t dequant8_zp(uint32_t w, half2_t s2, uint32_t magic,
                                               half2_t klo, half2_t khi)
{
    const uint32_t w8 = w >> 8;
    const half2_t s16 = {(f16)0.0625f, (f16)0.0625f};
    half2_t q[4];
    q[0] = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) | magic) + klo;
    q[1] = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) | magic) * s16 + khi;
    q[2] = __builtin_bit_cast(half2_t, (w8 & 0x000F000Fu) | magic) + klo;
    q[3] = __builtin_bit_cast(half2_t, (w8 & 0x00F000F0u) | magic) * s16 + khi;
    half8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t v = q[i] * s2;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

// The two offsets of zero point z as half2 pairs.
__device__ __forceinline__ void zp_offsets(uint32_t z, half2_t &klo, half2_t &khi)
{
    const f16 lo = (f16)(-1024.0f - (float)z), hi = (f16)(-64.0f - (float)z);
    klo = half2_t{lo, lo};
    khi = half2_t{hi, hi};
}

}  // namespace moe
