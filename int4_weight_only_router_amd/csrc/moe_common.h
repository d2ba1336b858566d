// moe_common.h -- internal helpers of libmoe_w4a16 (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "moe_w4a16.h"

namespace moe {

// Layout flags of the decode partials passed to the decode kernel: rows in
// token order, columns in partial-major order (MOE_Y_PARTIAL_ORDER).
constexpr int YF_TOKEN_ORDER = 1, YF_PARTIAL_ORDER = 2;

// Routed ids of one token mirrored into coherent pinned host memory by the
// routing kernel: ids[0..k) in rank order, then -- after a system-scope
// release -- *flag = seq, so a host thread that sees the flag sees the ids
// (no device-to-host copy, no event).  ids == nullptr: no mirror.
struct HostMirror {
    int32_t *ids;
    unsigned *flag;
    unsigned seq;
};

// Routing of one decode token formed inside the expert FFN from the logit
// partials of the fused combine (partial j of expert e at part[j * 64 + e];
// rows j >= min(64, H / 8) absent, taken as zero), plus the router's bias,
// flags and the routing outputs it writes.
struct DecodeRoute {
    const float *part;
    const float *bias;
    unsigned flags;
    int32_t *idx, *counts, *offsets, *perm, *inv_perm;
    float *w;
};

inline int decode_yflags(int regime)
{
    return ((regime & MOE_Y_TOKEN_ORDER) ? YF_TOKEN_ORDER : 0) |
           ((regime & MOE_Y_PARTIAL_ORDER) ? YF_PARTIAL_ORDER : 0);
}

// Partial-major column order: with C = H/8 chunks of 8 columns and
// q = ceil(C/64), column c of chunk u = 64m + j (j < 64) is stored at column
// 8(jq + m) + c mod 8.  A bijection when C <= 64 (then the identity) or C is
// a multiple of 64.
inline bool partial_order_ok(int H)
{
    const int C = H / 8;
    return H > 0 && H % 8 == 0 && (C <= 64 || C % 64 == 0);
}
__host__ __device__ inline int pm_col(int c, int H)
{
    const int q = (H / 8 + 63) / 64;
    const int u = c >> 3;
    return (((u & 63) * q + (u >> 6)) << 3) | (c & 7);
}

// ------------------------------------------------------------ errors (host)

int set_error(int code, const char *fmt, ...);   // stores a thread-local message
void clear_error();

#define MOE_HIP_TRY(expr)                                                        \
    do {                                                                         \
        hipError_t _e = (expr);                                                  \
        if (_e != hipSuccess)                                                    \
            return ::moe::set_error(MOE_EHIP, "%s failed: %s (%d)", #expr,        \
                                    hipGetErrorString(_e), (int)_e);             \
    } while (0)

// Launch check: a bad launch configuration is reported by hipGetLastError.
#define MOE_LAUNCH_CHECK(what)                                                   \
    do {                                                                         \
        hipError_t _e = hipGetLastError();                                       \
        if (_e != hipSuccess)                                                    \
            return ::moe::set_error(MOE_EHIP, "launch of %s failed: %s (%d)",     \
                                    what, hipGetErrorString(_e), (int)_e);       \
    } while (0)

inline int64_t al256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Shared-expert workspace (k_ffn_grouped.hip): its size, and where h starts.
size_t shared_ffn_ws_bytes(int T, int H, int Is);
_Float16 *shared_ffn_h(void *ws);

// Blob formats: symmetric codes (W = (u - 8) s) or a zero point per group
// (W = (u - z) s, one u8 per group of each projection after the scales).
enum { FMT_SYM = 0, FMT_ZP = 1 };

// Canonical blob section offsets (format documented in moe_w4a16.h); the
// zero-point sections exist only for FMT_ZP (else 0).
struct CanonLayout {
    int64_t gate_q, up_q, down_q, gate_s, up_s, down_s, gate_z, up_z, down_z, total;
};
inline CanonLayout canon_layout(int H, int I, int g, int fmt = FMT_SYM) {
    CanonLayout L;
    int64_t o = 0;
    L.gate_q = o; o = al256(o + int64_t(I) * H / 2);
    L.up_q = o;   o = al256(o + int64_t(I) * H / 2);
    L.down_q = o; o = al256(o + int64_t(H) * I / 2);
    L.gate_s = o; o = al256(o + int64_t(I) * (H / g) * 2);
    L.up_s = o;   o = al256(o + int64_t(I) * (H / g) * 2);
    L.down_s = o; o = al256(o + int64_t(H) * (I / g) * 2);
    L.gate_z = L.up_z = L.down_z = 0;
    if (fmt == FMT_ZP) {
        L.gate_z = o; o = al256(o + int64_t(I) * (H / g));
        L.up_z = o;   o = al256(o + int64_t(I) * (H / g));
        L.down_z = o; o = al256(o + int64_t(H) * (I / g));
    }
    L.total = o;
    return L;
}

// Device (prepacked) layout inside a blob of the same total size:
//   gu_q : fused gate/up INT4, I/32 blocks x (H/32 chunks) x 64 rows x 16 B
//   d_q  : down INT4, H/64 blocks x (I/32 chunks) x 64 rows x 16 B
//   gu_s : fused gate/up scales, I/32 blocks x (H/g) x 64 rows fp16
//   d_s  : down scales, H/64 blocks x (I/g) x 64 rows fp16
//   gu_z, d_z (FMT_ZP only): zero points in the scales' order, u8
struct DevLayout {
    int64_t gu_q, d_q, gu_s, d_s, gu_z, d_z, end;
};
inline DevLayout dev_layout(int H, int I, int g, int fmt = FMT_SYM) {
    DevLayout L;
    int64_t o = 0;
    L.gu_q = o; o = al256(o + int64_t(I) * H);
    L.d_q = o;  o = al256(o + int64_t(H) * I / 2);
    L.gu_s = o; o = al256(o + int64_t(2) * I * (H / g) * 2);
    L.d_s = o;  o = o + int64_t(H) * (I / g) * 2;
    L.gu_z = L.d_z = 0;
    if (fmt == FMT_ZP) {
        o = al256(o);
        L.gu_z = o; o = al256(o + int64_t(2) * I * (H / g));
        L.d_z = o;  o = o + int64_t(H) * (I / g);
    }
    L.end = o;
    return L;
}

// Shape envelope shared by the expert kernels.
inline bool h_supported(int H) {
    return H == 256 || H == 512 || H == 1024 || H == 2048;
}

// ------------------------------------------------------------- device side

typedef _Float16 f16;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt) but not for its outstanding global loads or stores, which a
// __syncthreads fence would drain first.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Loads through the global address space (plain pointers derived from a
// loaded blob address would otherwise become flat loads, which the hardware
// also counts against the LDS wait counter).
template <typename T>
__device__ __forceinline__ T ldg(const T *p)
{
    typedef const __attribute__((address_space(1))) T gT;
    return *(gT *)(p);
}

// Orders this wave's earlier LDS writes before its later LDS reads (LDS
// serves one wave's requests in order); no other wave is involved.
__device__ __forceinline__ void wave_lds_sync()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// SiLU(g) * u with the hardware exp2 / reciprocal (about 1 ulp each in fp32;
// the result is rounded to fp16).
__device__ __forceinline__ float swiglu_fast(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * g);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// The same with the non-temporal hint: for data streamed once per use that
// does not fit the last-level cache anyway (expert weights), so that it does
// not evict the small data that does (router weights, tables, activations).
template <typename T>
__device__ __forceinline__ T ldg_nt(const T *p)
{
    typedef const __attribute__((address_space(1))) T gT;
    return __builtin_nontemporal_load((gT *)p);
}

// Sum of one fp32 value per lane over the wave, in a fixed order: quad
// swaps (xor 1, xor 2), the half-row and row mirrors (register moves inside
// each 16-lane row; after the quad steps a mirror pairs whole quads and
// 8-lane halves), then the four row sums in row order.  Every lane gets the
// result.  For sums that decide no discrete choice (the pinned router order
// keeps its own butterfly).
template <int CTRL>
__device__ __forceinline__ float dpp_add_step(float a)
{
    return a + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                              0, __builtin_bit_cast(int, a), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_f32(float a)
{
    a = dpp_add_step<0xB1>(a);    // quad_perm [1,0,3,2]
    a = dpp_add_step<0x4E>(a);    // quad_perm [2,3,0,1]
    a = dpp_add_step<0x141>(a);   // row_half_mirror
    a = dpp_add_step<0x140>(a);   // row_mirror
    const int ai = __builtin_bit_cast(int, a);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ai, 48));
    return (r0 + r1) + (r2 + r3);
}

// Direct-to-LDS loads (global_load_lds): lane i's bytes land at the
// wave-uniform LDS address l + i * size; completion is counted by vmcnt.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const void *g, unsigned char *l)
{
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, unsigned char *l)
{
    __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 4, 0, 0);
}

// Waits until at most N vector-memory instructions of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float h2f(uint16_t bits) {
    return (float)__builtin_bit_cast(f16, bits);
}

}  // namespace moe
