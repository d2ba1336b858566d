// prepack_host.cpp -- the canonical <-> device blob bijection on the host
// (moe_prepack_expert_host / moe_unpack_expert_host): the same mapping as the
// device prepack kernel, for sources that live in host memory (the pinned
// INT4 source of the slot pool) so that no device round trip is needed.
#include <cstring>

#include "moe_common.h"

namespace moe {

int set_error(int code, const char *fmt, ...);
void clear_error();

// Canonical 32-bit word (element i at bits 4i) -> device word (element 2i at
// bits 4i, element 2i+1 at bits 16+4i), and back.
static uint32_t host_canon_to_dev(uint32_t cw)
{
    uint32_t d = 0;
    for (int i = 0; i < 4; ++i) {
        d |= ((cw >> (8 * i)) & 0xFu) << (4 * i);
        d |= ((cw >> (8 * i + 4)) & 0xFu) << (16 + 4 * i);
    }
    return d;
}

static uint32_t host_dev_to_canon(uint32_t dw)
{
    uint32_t c = 0;
    for (int i = 0; i < 4; ++i) {
        c |= ((dw >> (4 * i)) & 0xFu) << (8 * i);
        c |= ((dw >> (16 + 4 * i)) & 0xFu) << (8 * i + 4);
    }
    return c;
}

// One 16-byte chunk: dwords 1 and 2 trade places, each dword re-laid.
static void move_chunk(const uint8_t *s, uint8_t *d, bool to_dev)
{
    uint32_t v[4], o[4];
    std::memcpy(v, s, 16);
    const int order[4] = {0, 2, 1, 3};
    for (int i = 0; i < 4; ++i)
        o[i] = to_dev ? host_canon_to_dev(v[order[i]]) : host_dev_to_canon(v[order[i]]);
    std::memcpy(d, o, 16);
}

static int host_bijection(const char *fn, const void *src, int H, int I, int g, int fmt,
                          void *dst, bool to_dev)
{
    clear_error();
    if (!src || !dst)
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    if (H <= 0 || I <= 0 || g <= 0 || g % 32 || H % g || I % g || H % 64 || I % 32)
        return set_error(MOE_EINVAL, "%s: bad shape H=%d I=%d g=%d", fn, H, I, g);
    if (fmt != FMT_SYM && fmt != FMT_ZP)
        return set_error(MOE_EINVAL, "%s: unknown blob format %d", fn, fmt);
    const CanonLayout C = canon_layout(H, I, g, fmt);
    const DevLayout D = dev_layout(H, I, g, fmt);
    const uint8_t *s = static_cast<const uint8_t *>(src);
    uint8_t *d = static_cast<uint8_t *>(dst);
    if (s < d + C.total && d < s + C.total)
        return set_error(MOE_EINVAL, "%s: src and dst overlap", fn);
    std::memset(d, 0, (size_t)C.total);
    const int64_t NKH = H / 32, NKI = I / 32, HG = H / g, IG = I / g;
    // (canonical offset, device offset) of every piece, then the copy
    auto piece = [&](int64_t canoff, int64_t devoff, int kind) {
        const int64_t from = to_dev ? canoff : devoff, to = to_dev ? devoff : canoff;
        if (kind == 0)
            move_chunk(s + from, d + to, to_dev);
        else
            std::memcpy(d + to, s + from, (size_t)kind);
    };
    for (int64_t i = 0; i < (I / 32) * NKH * 64; ++i) {   // fused gate/up codes
        const int64_t b = i / (NKH * 64), c = (i / 64) % NKH, r = i % 64;
        piece((r < 32 ? C.gate_q : C.up_q) + (32 * b + (r & 31)) * (H / 2) + c * 16,
              D.gu_q + i * 16, 0);
    }
    for (int64_t j = 0; j < (H / 64) * NKI * 64; ++j) {   // down codes
        const int64_t b = j / (NKI * 64), c = (j / 64) % NKI, r = j % 64;
        piece(C.down_q + (64 * b + r) * (I / 2) + c * 16, D.d_q + j * 16, 0);
    }
    for (int64_t j = 0; j < (I / 32) * HG * 64; ++j) {    // gate/up scales (and zero points)
        const int64_t b = j / (HG * 64), G = (j / 64) % HG, r = j % 64;
        const int64_t cr = (32 * b + (r & 31)) * HG + G;
        piece((r < 32 ? C.gate_s : C.up_s) + cr * 2, D.gu_s + j * 2, 2);
        if (fmt == FMT_ZP)
            piece((r < 32 ? C.gate_z : C.up_z) + cr, D.gu_z + j, 1);
    }
    for (int64_t j = 0; j < (H / 64) * IG * 64; ++j) {    // down scales (and zero points)
        const int64_t b = j / (IG * 64), G = (j / 64) % IG, r = j % 64;
        const int64_t cr = (64 * b + r) * IG + G;
        piece(C.down_s + cr * 2, D.d_s + j * 2, 2);
        if (fmt == FMT_ZP)
            piece(C.down_z + cr, D.d_z + j, 1);
    }
    return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_prepack_expert_host(const void *src, int H, int I, int group, int fmt, void *dst)
{
    return moe::host_bijection("moe_prepack_expert_host", src, H, I, group, fmt, dst, true);
}

int moe_unpack_expert_host(const void *src, int H, int I, int group, int fmt, void *dst)
{
    return moe::host_bijection("moe_unpack_expert_host", src, H, I, group, fmt, dst, false);
}

}  // extern "C"
