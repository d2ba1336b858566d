// k_quant.hip -- load-time INT4 quantisation and the canonical <-> device
// layout bijection of expert blobs.
//
// Horizon RunMap "08 / Comportamento do modelo": routed expert weights are
// stored as INT4 with FP16 scales; lucashiago.com.br explainer, step 1: each
// block of weights carries its scale (and, in the zero-point format, its zero
// point).  Reading: groups of g along the input dimension; symmetric:
// s = fp16_rne(amax / 7) with amax / 7 in fp32, q = clamp(rne(w / s), -7, 7)
// with w / s in fp32, q = 0 when s = 0, stored as u = q + 8; zero point: see
// quantize_rows_kernel.  Element 2b in the low nibble of byte b.
#include <algorithm>

#include "moe_common.h"

namespace moe {

// One thread per 32-element chunk of a row; a group of g spans g/32 adjacent
// threads of one wave, which share the group's extremes through lane
// shuffles.  ZP: the zero-point format (reading: lo = min(min w, 0),
// hi = max(max w, 0), s = fp16_rne((hi - lo) / 15), z = clamp(rne(-lo / s),
// 0, 15), u = clamp(rne(w / s) + z, 0, 15); s = 0 gives z = u = 0; the
// quotients in fp32); off_z receives one byte per group.
template <bool ZP>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const float *__restrict__ w, int64_t w_stride, int rows, int K, int g,
    uint8_t *__restrict__ blobs, int64_t blob_stride, int64_t off_q, int64_t off_s, int64_t off_z)
{
    const int n = blockIdx.y;
    const int nch = K / 32;
    const int64_t cid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool valid = cid < (int64_t)rows * nch;
    const int row = valid ? (int)(cid / nch) : 0;
    const int c = valid ? (int)(cid % nch) : 0;
    const float *src = w + n * w_stride + (int64_t)row * K + c * 32;
    float v[32];
    float amax = 0.0f, lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4_t f = valid ? *reinterpret_cast<const float4_t *>(src + 4 * i)
                           : float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            v[4 * i + m] = f[m];
            amax = fmaxf(amax, fabsf(f[m]));
            lo = fminf(lo, f[m]);
            hi = fmaxf(hi, f[m]);
        }
    }
    const int span = g / 32;   // 1, 2 or 4 threads per group
    for (int st = 1; st < span; st <<= 1) {
        amax = fmaxf(amax, __shfl_xor(amax, st, 64));
        lo = fminf(lo, __shfl_xor(lo, st, 64));
        hi = fmaxf(hi, __shfl_xor(hi, st, 64));
    }
    if (!valid)
        return;
    const f16 sh = ZP ? (f16)((hi - lo) / 15.0f) : (f16)(amax / 7.0f);
    const float sv = (float)sh;
    int zi = 8;   // symmetric: u = q + 8
    if (ZP)
        zi = sv != 0.0f ? (int)fminf(fmaxf(rintf(-lo / sv), 0.0f), 15.0f) : 0;
    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        int u = 0;
        if (sv != 0.0f) {
            const float r = rintf(v[i] / sv);
            u = ZP ? (int)fminf(fmaxf(r + (float)zi, 0.0f), 15.0f)
                   : (int)fminf(fmaxf(r, -7.0f), 7.0f) + 8;
        } else {
            u = ZP ? 0 : 8;
        }
        words[i >> 3] |= (uint32_t)u << (4 * (i & 7));   // canonical: element i at bits 4i
    }
    uint8_t *blob = blobs + n * blob_stride;
    *reinterpret_cast<uint4_t *>(blob + off_q + (int64_t)row * (K / 2) + c * 16) =
        uint4_t{words[0], words[1], words[2], words[3]};
    if ((c * 32) % g == 0) {
        reinterpret_cast<f16 *>(blob + off_s)[(int64_t)row * (K / g) + (c * 32) / g] = sh;
        if (ZP)
            blob[off_z + (int64_t)row * (K / g) + (c * 32) / g] = (uint8_t)zi;
    }
}

__device__ __forceinline__ uint32_t canon_to_dev(uint32_t cw)
{
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d |= ((cw >> (8 * i)) & 0xFu) << (4 * i);
        d |= ((cw >> (8 * i + 4)) & 0xFu) << (16 + 4 * i);
    }
    return d;
}

__device__ __forceinline__ uint32_t dev_to_canon(uint32_t dw)
{
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c |= ((dw >> (4 * i)) & 0xFu) << (8 * i);
        c |= ((dw >> (16 + 4 * i)) & 0xFu) << (8 * i + 4);
    }
    return c;
}

__global__ __launch_bounds__(256) void zero_kernel(uint4_t *p, int64_t n16)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = uint4_t{0u, 0u, 0u, 0u};
}

// Byte-granular zero fill (any address and size): 16-byte stores over the
// aligned middle, single bytes at the ends.
__global__ __launch_bounds__(256) void zero_bytes_kernel(uint8_t *p, int64_t head, int64_t n16,
                                                         int64_t tail)
{
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = tid; i < head; i += stride)
        p[i] = 0;
    uint4_t *m = reinterpret_cast<uint4_t *>(p + head);
    for (int64_t i = tid; i < n16; i += stride)
        m[i] = uint4_t{0u, 0u, 0u, 0u};
    uint8_t *t = p + head + 16 * n16;
    for (int64_t i = tid; i < tail; i += stride)
        t[i] = 0;
}

int launch_zero_bytes(void *p, size_t bytes, hipStream_t s)
{
    if (bytes == 0)
        return MOE_OK;
    uint8_t *b = static_cast<uint8_t *>(p);
    int64_t head = (int64_t)((16 - (reinterpret_cast<uintptr_t>(b) & 15)) & 15);
    if (head > (int64_t)bytes)
        head = (int64_t)bytes;
    const int64_t n16 = ((int64_t)bytes - head) / 16;
    const int64_t tail = (int64_t)bytes - head - 16 * n16;
    const int64_t work = std::max<int64_t>(std::max(head, tail), n16);
    const unsigned blocks = (unsigned)std::min<int64_t>(1024, (work + 255) / 256);
    hipLaunchKernelGGL(zero_bytes_kernel, dim3(blocks), dim3(256), 0, s, b, head, n16, tail);
    MOE_LAUNCH_CHECK("zero_bytes_kernel");
    return MOE_OK;
}

// Item ranges: [0,nguq) fused gate/up 16-byte chunks, then down chunks, then
// fused gate/up scales, then down scales.  dir = 0: canonical -> device.
// Inside a device chunk word the four dwords hold elements 0-7, 16-23, 8-15,
// 24-31 of the chunk: bytes 0-7 are then the K-half one MFMA lane group needs
// for two consecutive 16-K steps, bytes 8-15 the other half.
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t *__restrict__ src,
                                                      uint8_t *__restrict__ dst, int H, int I,
                                                      int g, int64_t stride, CanonLayout C,
                                                      DevLayout D, int dir, int zp)
{
    const int n = blockIdx.y;
    const int NKH = H / 32, NKI = I / 32, HG = H / g, IG = I / g;
    const int64_t nguq = (int64_t)(I / 32) * NKH * 64;
    const int64_t ndq = (int64_t)(H / 64) * NKI * 64;
    const int64_t ngus = (int64_t)(I / 32) * HG * 64;
    const int64_t nds = (int64_t)(H / 64) * IG * 64;
    const int64_t nsec = nguq + ndq + ngus + nds;
    const int64_t ntot = nsec + (zp ? ngus + nds : 0);   // zero points: one byte per scale
    const uint8_t *s = src + n * stride;
    uint8_t *d = dst + n * stride;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ntot;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t devoff, canoff;
        int kind;   // 0 = 16-byte nibble chunk, 1 = 2-byte scale, 2 = 1-byte zero point
        if (i < nguq) {
            const int64_t b = i / (NKH * 64), c = (i / 64) % NKH, r = i % 64;
            const int64_t row = 32 * b + (r & 31);
            devoff = D.gu_q + i * 16;
            canoff = (r < 32 ? C.gate_q : C.up_q) + row * (H / 2) + c * 16;
            kind = 0;
        } else if (i < nguq + ndq) {
            const int64_t j = i - nguq;
            const int64_t b = j / (NKI * 64), c = (j / 64) % NKI, r = j % 64;
            devoff = D.d_q + j * 16;
            canoff = C.down_q + (64 * b + r) * (I / 2) + c * 16;
            kind = 0;
        } else if (i < nguq + ndq + ngus || (i >= nsec && i < nsec + ngus)) {
            const bool z = i >= nsec;
            const int64_t j = z ? i - nsec : i - nguq - ndq;
            const int64_t b = j / (HG * 64), G = (j / 64) % HG, r = j % 64;
            const int64_t cr = (32 * b + (r & 31)) * HG + G;
            devoff = z ? D.gu_z + j : D.gu_s + j * 2;
            canoff = z ? (r < 32 ? C.gate_z : C.up_z) + cr
                       : (r < 32 ? C.gate_s : C.up_s) + cr * 2;
            kind = z ? 2 : 1;
        } else {
            const bool z = i >= nsec;
            const int64_t j = z ? i - nsec - ngus : i - nguq - ndq - ngus;
            const int64_t b = j / (IG * 64), G = (j / 64) % IG, r = j % 64;
            const int64_t cr = (64 * b + r) * IG + G;
            devoff = z ? D.d_z + j : D.d_s + j * 2;
            canoff = z ? C.down_z + cr : C.down_s + cr * 2;
            kind = z ? 2 : 1;
        }
        if (kind == 0) {
            // dwords 1 and 2 trade places (the swap is its own inverse)
            const uint4_t v = *reinterpret_cast<const uint4_t *>(s + (dir == 0 ? canoff : devoff));
            uint4_t o;
            if (dir == 0)
                o = uint4_t{canon_to_dev(v.x), canon_to_dev(v.z), canon_to_dev(v.y),
                            canon_to_dev(v.w)};
            else
                o = uint4_t{dev_to_canon(v.x), dev_to_canon(v.z), dev_to_canon(v.y),
                            dev_to_canon(v.w)};
            *reinterpret_cast<uint4_t *>(d + (dir == 0 ? devoff : canoff)) = o;
        } else if (kind == 1) {
            *reinterpret_cast<uint16_t *>(d + (dir == 0 ? devoff : canoff)) =
                *reinterpret_cast<const uint16_t *>(s + (dir == 0 ? canoff : devoff));
        } else {
            d[dir == 0 ? devoff : canoff] = s[dir == 0 ? canoff : devoff];
        }
    }
}

int launch_quantize(const float *wg, const float *wu, const float *wd, int n, int H, int I, int g,
                    int fmt, void *blobs, hipStream_t s)
{
    const CanonLayout C = canon_layout(H, I, g, fmt);
    uint8_t *b = static_cast<uint8_t *>(blobs);
    hipLaunchKernelGGL(zero_kernel, dim3(1024), dim3(256), 0, s, (uint4_t *)b,
                       (int64_t)n * C.total / 16);
    MOE_LAUNCH_CHECK("zero_kernel");
    struct P { const float *w; int rows, K; int64_t q, sc, z; } ps[3] = {
        {wg, I, H, C.gate_q, C.gate_s, C.gate_z}, {wu, I, H, C.up_q, C.up_s, C.up_z},
        {wd, H, I, C.down_q, C.down_s, C.down_z}};
    for (const P &p : ps) {
        const int64_t chunks = (int64_t)p.rows * (p.K / 32);
        dim3 grid((unsigned)((chunks + 255) / 256), n);
        if (fmt == FMT_ZP)
            hipLaunchKernelGGL(quantize_rows_kernel<true>, grid, dim3(256), 0, s, p.w,
                               (int64_t)p.rows * p.K, p.rows, p.K, g, b, C.total, p.q, p.sc, p.z);
        else
            hipLaunchKernelGGL(quantize_rows_kernel<false>, grid, dim3(256), 0, s, p.w,
                               (int64_t)p.rows * p.K, p.rows, p.K, g, b, C.total, p.q, p.sc,
                               (int64_t)0);
        MOE_LAUNCH_CHECK("quantize_rows_kernel");
    }
    return MOE_OK;
}

int launch_prepack(const void *src, int n, int H, int I, int g, int fmt, void *dst, int dir,
                   hipStream_t s)
{
    const CanonLayout C = canon_layout(H, I, g, fmt);
    const DevLayout D = dev_layout(H, I, g, fmt);
    hipLaunchKernelGGL(zero_kernel, dim3(1024), dim3(256), 0, s, (uint4_t *)dst,
                       (int64_t)n * C.total / 16);
    MOE_LAUNCH_CHECK("zero_kernel");
    hipLaunchKernelGGL(prepack_kernel, dim3(512, n), dim3(256), 0, s,
                       static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), H, I, g,
                       C.total, C, D, dir, fmt == FMT_ZP ? 1 : 0);
    MOE_LAUNCH_CHECK("prepack_kernel");
    return MOE_OK;
}

}  // namespace moe
