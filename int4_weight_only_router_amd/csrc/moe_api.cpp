// moe_api.cpp -- the C ABI of libmoe_w4a16: argument validation, regime
// choice and dispatch to the HIP kernels.  Nothing here computes on the host.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "moe_common.h"
#include "trace.h"

namespace moe {

static thread_local std::string g_err;

int set_error(int code, const char *fmt, ...)
{
    char buf[768];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

void clear_error() { g_err.clear(); }

// kernels (defined in the .hip files)
int launch_route(const void *, const void *, const float *, int, int, int, int, unsigned,
                 int32_t *, float *, hipStream_t);
size_t permute_ws_bytes(int T, int k, int E);
size_t route_split_ws_bytes(int T, int E);
size_t route_batched_ws_bytes(int T, int E);
int launch_route_batched(const void *, const void *, const float *, int, int, int, int, unsigned,
                         int32_t *, float *, void *, hipStream_t);
int launch_route_split_mirrored(const void *, const void *, const float *, int, int, int, unsigned,
                                int32_t *, float *, int32_t *, int32_t *, int32_t *, int32_t *,
                                void *, HostMirror, hipStream_t);
int launch_route_split(const void *, const void *, const float *, int, int, int, int, unsigned,
                       int32_t *, float *, int32_t *, int32_t *, int32_t *, int32_t *, void *,
                       hipStream_t);
int launch_permute(const int32_t *, int, int, int, int32_t *, int32_t *, int32_t *, int32_t *,
                   void *, hipStream_t);
int launch_ffn_decode(const void *, const int32_t *, const int32_t *, const void *const *,
                      const void *const *, int, int, int, int, int, int, int, int, float *,
                      hipStream_t, const DecodeRoute *);
size_t ffn_batched_ws_bytes(int T, int I, int k);
int launch_ffn_batched(const void *, const int32_t *, const int32_t *, const void *const *, int,
                       int, int, int, int, int, int, void *, void *, hipStream_t);
bool ffn_small_fits(int T, int H, int I);
int launch_ffn_small(const void *, const int32_t *, const int32_t *, const void *const *, int, int,
                     int, int, int, int, int, void *, void *, hipStream_t);
int launch_shared_gemv(const void *, const void *, const void *, const void *, int, int, int,
                       float *, void *, hipStream_t);
int launch_shared_batched(const void *, const void *, const void *, const void *, int, int, int,
                          float *, void *, hipStream_t);
int launch_combine_route(const float *, bool, int, const int32_t *, const float *, const float *,
                         const void *, const void *, const void *, int, int, void *,
                         const void *, const float *, int, int, unsigned, void *, int32_t *,
                         float *, int32_t *, int32_t *, int32_t *, int32_t *, float *,
                         hipStream_t);
size_t combine_route_ws_bytes();
int launch_logit_partials(const void *, const void *, int, int, float *, hipStream_t);
int launch_combine(const void *, int, int, const int32_t *, const float *, const float *,
                   const void *, const void *, const void *, int, int, int, void *,
                   hipStream_t);
int launch_quantize(const float *, const float *, const float *, int, int, int, int, int, void *,
                    hipStream_t);
int launch_prepack(const void *, int, int, int, int, int, void *, int, hipStream_t);
int launch_zero_bytes(void *, size_t, hipStream_t);

constexpr int DECODE_MAX_T = 4;       // AUTO: decode kernel up to this many tokens
constexpr int SMALL_MAX_T = 32;       // AUTO: small-batch kernel up to this many tokens
constexpr int ROUTE_FUSED_MAX_T = 5;  // moe_route_permute: one fused launch up to this T
// E > 128: the fused launch's single selecting workgroup takes every token's
// top-k in turn, so it pays only for the smallest T
constexpr int ROUTE_FUSED_MAX_T_BIGE = 4;

constexpr size_t ROUTE_TICKET_BYTES = 256;   // the fused router's arrival ticket, ws[0..256)

static bool route_fused(int T, int E)
{
    return T > 0 && T <= (E > 128 ? ROUTE_FUSED_MAX_T_BIGE : ROUTE_FUSED_MAX_T);
}
constexpr int ROUTE_SMALL_MAX_T = 8;  // moe_route: one-workgroup kernel up to this T

// Workspace of moe_route_permute_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is only a stand-in for the symbol): each
// device's address comes from hipGetSymbolAddress at set-up.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[MAX_DEVICES];

// This device's scratch address; on the first call on a device (with that
// device current) it is looked up and the fused router's ticket is cleared
// by a kernel on `stream`, ordered before the caller's launches.
static int noalloc_scratch(hipStream_t stream, void **out)
{
    int dev = -1;
    MOE_HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES)
        return set_error(MOE_EUNSUPPORTED, "moe_route_permute_noalloc: device %d out of range",
                         dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        MOE_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p)
            return set_error(MOE_EHIP, "moe_route_permute_noalloc: no address for the scratch");
        const int rc = launch_zero_bytes(p, ROUTE_TICKET_BYTES, stream);
        if (rc)
            return rc;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
constexpr int SHARED_GEMV_MAX_T = 8;  // shared expert: GEMV up to this many tokens

static int check_expert_shape(const char *fn, int H, int I, int g)
{
    if (H <= 0 || I <= 0 || g <= 0)
        return set_error(MOE_EINVAL, "%s: non-positive size (H=%d I=%d g=%d)", fn, H, I, g);
    if (g % 32 || H % g || I % g)
        return set_error(MOE_EINVAL, "%s: group %d must be a multiple of 32 dividing H=%d, I=%d",
                         fn, g, H, I);
    if (!h_supported(H) || I % 64 || I > 8192 || (g != 32 && g != 64 && g != 128))
        return set_error(MOE_EUNSUPPORTED,
                         "%s: outside the kernel envelope (H in {256, 512, 1024, 2048}, "
                         "I %% 64 == 0 and <= 8192, g in {32,64,128}); got H=%d I=%d g=%d",
                         fn, H, I, g);
    return MOE_OK;
}

static int check_route_shape(const char *fn, int T, int E, int k)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E)
        return set_error(MOE_EINVAL, "%s: need T >= 0, E > 0, 0 < k <= E (T=%d E=%d k=%d)", fn,
                         T, E, k);
    if (E > 1024 || k > 16)
        return set_error(MOE_EUNSUPPORTED, "%s: E <= 1024 and k <= 16 required (E=%d k=%d)", fn,
                         E, k);
    if ((int64_t)T * k >= (int64_t)1 << 31)
        return set_error(MOE_EUNSUPPORTED, "%s: T*k too large", fn);
    return MOE_OK;
}

static int resolve_regime(int T, int H, int I, int regime)
{
    if (regime == MOE_REGIME_AUTO) {
        if (T <= DECODE_MAX_T)
            return MOE_REGIME_DECODE;
        if (T <= SMALL_MAX_T && ffn_small_fits(T, H, I))
            return MOE_REGIME_SMALL;
        return MOE_REGIME_BATCHED;
    }
    return regime;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

int moe_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    if (ws_bytes == 0)
        return MOE_OK;
    if (!ws)
        return set_error(MOE_EINVAL, "moe_workspace_clear: null workspace");
    return launch_zero_bytes(ws, ws_bytes, stream);
}

int moe_blob_layout_fmt(int H, int I, int group, int fmt, int64_t offsets[9],
                        int64_t *total_bytes)
{
    clear_error();
    if (!offsets || !total_bytes || H <= 0 || I <= 0 || group <= 0 || H % group || I % group ||
        H % 2 || I % 2 || (fmt != MOE_FMT_SYM && fmt != MOE_FMT_ZP))
        return set_error(MOE_EINVAL, "moe_blob_layout_fmt: bad arguments (H=%d I=%d g=%d fmt=%d)",
                         H, I, group, fmt);
    const CanonLayout L = canon_layout(H, I, group, fmt);
    const int64_t o[9] = {L.gate_q, L.up_q, L.down_q, L.gate_s, L.up_s, L.down_s,
                          L.gate_z, L.up_z, L.down_z};
    for (int i = 0; i < 9; ++i)
        offsets[i] = o[i];
    *total_bytes = L.total;
    return MOE_OK;
}

int moe_blob_layout(int H, int I, int group, int64_t offsets[6], int64_t *total_bytes)
{
    int64_t o[9];
    if (!offsets)
        return set_error(MOE_EINVAL, "moe_blob_layout: null offsets");
    const int rc = moe_blob_layout_fmt(H, I, group, MOE_FMT_SYM, o, total_bytes);
    if (rc)
        return rc;
    for (int i = 0; i < 6; ++i)
        offsets[i] = o[i];
    return MOE_OK;
}

static int check_fmt(const char *fn, int fmt)
{
    if (fmt != MOE_FMT_SYM && fmt != MOE_FMT_ZP)
        return set_error(MOE_EINVAL, "%s: unknown blob format %d", fn, fmt);
    return MOE_OK;
}

int moe_quantize_experts_fmt(const float *wg, const float *wu, const float *wd, int n, int H,
                             int I, int group, int fmt, void *blobs, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    if (!wg || !wu || !wd || !blobs || n < 0)
        return set_error(MOE_EINVAL, "moe_quantize_experts: null pointer or n < 0");
    int rc = check_fmt("moe_quantize_experts", fmt);
    if (!rc)
        rc = check_expert_shape("moe_quantize_experts", H, I, group);
    if (rc || n == 0)
        return rc;
    return launch_quantize(wg, wu, wd, n, H, I, group, fmt, blobs, stream);
}

int moe_quantize_experts(const float *wg, const float *wu, const float *wd, int n, int H, int I,
                         int group, void *blobs, hipStream_t stream)
{
    MOE_API_RANGE();
    return moe_quantize_experts_fmt(wg, wu, wd, n, H, I, group, MOE_FMT_SYM, blobs, stream);
}

static int prepack_common(const char *fn, const void *src, int n, int H, int I, int group,
                          int fmt, void *dst, int dir, hipStream_t stream)
{
    clear_error();
    if (!src || !dst || n < 0)
        return set_error(MOE_EINVAL, "%s: null pointer or n < 0", fn);
    int rc = check_fmt(fn, fmt);
    if (!rc)
        rc = check_expert_shape(fn, H, I, group);
    if (rc || n == 0)
        return rc;
    const int64_t tot = canon_layout(H, I, group, fmt).total * (int64_t)n;
    const char *a = static_cast<const char *>(src), *b = static_cast<const char *>(dst);
    if (a < b + tot && b < a + tot)
        return set_error(MOE_EINVAL, "%s: src and dst overlap", fn);
    return launch_prepack(src, n, H, I, group, fmt, dst, dir, stream);
}

int moe_prepack_experts(const void *src, int n, int H, int I, int group, void *dst,
                        hipStream_t stream)
{
    MOE_API_RANGE();
    return prepack_common("moe_prepack_experts", src, n, H, I, group, MOE_FMT_SYM, dst, 0,
                          stream);
}

int moe_unpack_experts(const void *src, int n, int H, int I, int group, void *dst,
                       hipStream_t stream)
{
    MOE_API_RANGE();
    return prepack_common("moe_unpack_experts", src, n, H, I, group, MOE_FMT_SYM, dst, 1, stream);
}

int moe_prepack_experts_fmt(const void *src, int n, int H, int I, int group, int fmt, void *dst,
                            hipStream_t stream)
{
    MOE_API_RANGE();
    return prepack_common("moe_prepack_experts_fmt", src, n, H, I, group, fmt, dst, 0, stream);
}

int moe_unpack_experts_fmt(const void *src, int n, int H, int I, int group, int fmt, void *dst,
                           hipStream_t stream)
{
    MOE_API_RANGE();
    return prepack_common("moe_unpack_experts_fmt", src, n, H, I, group, fmt, dst, 1, stream);
}

static int check_route_args(const char *fn, const void *x_f16, const void *w_router_f16, int T,
                            int H, int E, int k, unsigned flags, const int32_t *topk_idx,
                            const float *topk_w)
{
    int rc = check_route_shape(fn, T, E, k);
    if (rc)
        return rc;
    if (T > 0 && (!x_f16 || !w_router_f16 || !topk_idx || !topk_w))
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    if (H <= 0 || H % 8)
        return set_error(MOE_EINVAL, "%s: H=%d must be a positive multiple of 8", fn, H);
    if (!h_supported(H))
        return set_error(MOE_EUNSUPPORTED, "%s: H=%d not in {256, 512, 1024, 2048}", fn, H);
    if (flags & ~(unsigned)MOE_RENORM)
        return set_error(MOE_EINVAL, "%s: unknown flags 0x%x", fn, flags);
    return MOE_OK;
}

size_t moe_route_workspace_bytes(int T, int E)
{
    if (T <= ROUTE_SMALL_MAX_T || E <= 0)
        return 0;
    return route_batched_ws_bytes(T, E);
}

int moe_route(const void *x_f16, const void *w_router_f16, const float *logit_bias, int T, int H,
              int E, int k, unsigned flags, int32_t *topk_idx, float *topk_w, void *ws,
              size_t ws_bytes, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    int rc = check_route_args("moe_route", x_f16, w_router_f16, T, H, E, k, flags, topk_idx,
                              topk_w);
    if (rc)
        return rc;
    if (T <= ROUTE_SMALL_MAX_T)
        return launch_route(x_f16, w_router_f16, logit_bias, T, H, E, k, flags, topk_idx, topk_w,
                            stream);
    const size_t need = moe_route_workspace_bytes(T, E);
    if (!ws || ws_bytes < need)
        return set_error(MOE_ENOMEM, "moe_route: workspace %zu < %zu bytes", ws_bytes, need);
    return launch_route_batched(x_f16, w_router_f16, logit_bias, T, H, E, k, flags, topk_idx,
                                topk_w, ws, stream);
}

size_t moe_route_permute_workspace_bytes(int T, int k, int E)
{
    if (T < 0 || k <= 0 || E <= 0)
        return 0;
    if (route_fused(T, E))
        return route_split_ws_bytes(T, E);
    // the fused launch's ticket (left zero), logits of the batched router,
    // then the permutation's scratch
    return ROUTE_TICKET_BYTES + route_batched_ws_bytes(T, E) + permute_ws_bytes(T, k, E);
}

}  // extern "C"

namespace moe {
// moe_route_permute; with a host mirror (hm.ids set) and one token of at most
// 64 experts, the fused launch also writes the routed ids and the mirror's
// flag into host memory (*mirrored = true).
int route_permute_mirror(const void *x_f16, const void *w_router_f16, const float *logit_bias,
                         int T, int H, int E, int k, unsigned flags, int32_t *topk_idx,
                         float *topk_w, int32_t *counts, int32_t *offsets, int32_t *perm,
                         int32_t *inv_perm, void *ws, size_t ws_bytes, HostMirror hm,
                         bool *mirrored, hipStream_t stream)
{
    *mirrored = false;
    int rc = check_route_args("moe_route_permute", x_f16, w_router_f16, T, H, E, k, flags,
                              topk_idx, topk_w);
    if (rc)
        return rc;
    if (!counts || !offsets || (T > 0 && (!perm || !inv_perm)))
        return set_error(MOE_EINVAL, "moe_route_permute: null pointer");
    const size_t need = moe_route_permute_workspace_bytes(T, k, E);
    if (need && (!ws || ws_bytes < need))
        return set_error(MOE_ENOMEM, "moe_route_permute: workspace %zu < %zu bytes", ws_bytes,
                         need);
    if (hm.ids && T == 1 && E <= 64 && k <= 64 && route_fused(T, E)) {
        *mirrored = true;
        return launch_route_split_mirrored(x_f16, w_router_f16, logit_bias, H, E, k, flags,
                                           topk_idx, topk_w, counts, offsets, perm, inv_perm, ws,
                                           hm, stream);
    }
    if (route_fused(T, E))
        return launch_route_split(x_f16, w_router_f16, logit_bias, T, H, E, k, flags, topk_idx,
                                  topk_w, counts, offsets, perm, inv_perm, ws, stream);
    void *pws = nullptr;
    if (T > 0) {
        // past the ticket, so one workspace serves batches on both sides of
        // the fused/batched boundary
        char *lws = static_cast<char *>(ws) + ROUTE_TICKET_BYTES;
        rc = launch_route_batched(x_f16, w_router_f16, logit_bias, T, H, E, k, flags, topk_idx,
                                  topk_w, lws, stream);
        if (rc)
            return rc;
        pws = lws + route_batched_ws_bytes(T, E);
    }
    return launch_permute(topk_idx, T, k, E, counts, offsets, perm, inv_perm, pws, stream);
}
}  // namespace moe

extern "C" {

int moe_route_permute(const void *x_f16, const void *w_router_f16, const float *logit_bias, int T,
                      int H, int E, int k, unsigned flags, int32_t *topk_idx, float *topk_w,
                      int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                      void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    bool mirrored = false;
    return route_permute_mirror(x_f16, w_router_f16, logit_bias, T, H, E, k, flags, topk_idx,
                                topk_w, counts, offsets, perm, inv_perm, ws, ws_bytes,
                                HostMirror{nullptr, nullptr, 0u}, &mirrored, stream);
}

int moe_route_permute_noalloc(const void *x_f16, const void *w_router_f16,
                              const float *logit_bias, int T, int H, int E, int k, unsigned flags,
                              int32_t *topk_idx, float *topk_w, int32_t *counts, int32_t *offsets,
                              int32_t *perm, int32_t *inv_perm, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    int rc = check_route_args("moe_route_permute_noalloc", x_f16, w_router_f16, T, H, E, k,
                              flags, topk_idx, topk_w);
    if (rc)
        return rc;
    if (!counts || !offsets || (T > 0 && (!perm || !inv_perm)))
        return set_error(MOE_EINVAL, "moe_route_permute_noalloc: null pointer");
    const size_t need = moe_route_permute_workspace_bytes(T, k, E);
    if (need > NOALLOC_SCRATCH_BYTES)
        return set_error(MOE_ENOMEM,
                         "moe_route_permute_noalloc: T=%d E=%d k=%d needs %zu bytes of scratch; "
                         "the library holds %zu (use moe_route_permute with a workspace)",
                         T, E, k, need, NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    rc = noalloc_scratch(stream, &ws);
    if (rc)
        return rc;
    return moe_route_permute(x_f16, w_router_f16, logit_bias, T, H, E, k, flags, topk_idx, topk_w,
                             counts, offsets, perm, inv_perm, ws, NOALLOC_SCRATCH_BYTES, stream);
}

size_t moe_permute_workspace_bytes(int T, int k, int E)
{
    if (T < 0 || k <= 0 || E <= 0)
        return 0;
    return permute_ws_bytes(T, k, E);
}

int moe_permute(const int32_t *topk_idx, int T, int k, int E, int32_t *counts, int32_t *offsets,
                int32_t *perm, int32_t *inv_perm, void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    int rc = check_route_shape("moe_permute", T, E, k);
    if (rc)
        return rc;
    if (!counts || !offsets || (T > 0 && (!topk_idx || !perm || !inv_perm)))
        return set_error(MOE_EINVAL, "moe_permute: null pointer");
    const size_t need = permute_ws_bytes(T, k, E);
    if (need && (!ws || ws_bytes < need))
        return set_error(MOE_ENOMEM, "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);
    return launch_permute(topk_idx, T, k, E, counts, offsets, perm, inv_perm, ws, stream);
}

int moe_expert_ffn_plan(int T, int H, int I, int E, int k, int group, int regime,
                        int *resolved_regime, int *y_dtype, int *y_slices, size_t *ws_bytes)
{
    clear_error();
    int rc = check_route_shape("moe_expert_ffn_plan", T, E, k);
    if (rc)
        return rc;
    rc = check_expert_shape("moe_expert_ffn_plan", H, I, group);
    if (rc)
        return rc;
    const bool tok = (regime & MOE_Y_TOKEN_ORDER) != 0;
    const bool pm = (regime & MOE_Y_PARTIAL_ORDER) != 0;
    regime &= ~(MOE_Y_TOKEN_ORDER | MOE_Y_PARTIAL_ORDER | MOE_W4_ZERO_POINT);
    if (regime < MOE_REGIME_AUTO || regime > MOE_REGIME_SMALL)
        return set_error(MOE_EINVAL, "moe_expert_ffn_plan: bad regime %d", regime);
    const int r = resolve_regime(T, H, I, regime);
    if ((tok || pm) && r != MOE_REGIME_DECODE)
        return set_error(MOE_EUNSUPPORTED,
                         "moe_expert_ffn_plan: token-order and partial-major y are "
                         "DECODE-regime options (resolved regime %d)", r);
    if (pm && !partial_order_ok(H))
        return set_error(MOE_EUNSUPPORTED,
                         "moe_expert_ffn_plan: H=%d has no partial-major column order", H);
    if (r == MOE_REGIME_SMALL && !ffn_small_fits(T, H, I))
        return set_error(MOE_EUNSUPPORTED,
                         "moe_expert_ffn_plan: small-batch regime takes T <= 32 (T=%d)", T);
    if (resolved_regime)
        *resolved_regime = r;
    if (y_dtype)
        *y_dtype = (r == MOE_REGIME_DECODE) ? (pm ? MOE_DTYPE_F32_PM : MOE_DTYPE_F32)
                                            : MOE_DTYPE_F16;
    if (y_slices)
        *y_slices = (r == MOE_REGIME_DECODE) ? I / 32 : 1;
    if (ws_bytes)
        *ws_bytes = (r == MOE_REGIME_DECODE) ? 0 : ffn_batched_ws_bytes(T, I, k);
    return MOE_OK;
}

int moe_expert_ffn_w4a16(const void *x_f16, const int32_t *perm, const int32_t *offsets,
                         const void *const *d_expert_blobs, int T, int H, int I, int E, int k,
                         int group, int regime, void *y, int y_dtype, int y_slices, void *ws,
                         size_t ws_bytes, hipStream_t stream)
{
    MOE_API_RANGE();
    int r = 0, dt = 0, sl = 0;
    size_t need = 0;
    int rc = moe_expert_ffn_plan(T, H, I, E, k, group, regime, &r, &dt, &sl, &need);
    if (rc)
        return rc;
    if (y_dtype != dt || y_slices != sl)
        return set_error(MOE_EINVAL,
                         "moe_expert_ffn_w4a16: y must be dtype %d with %d slices for this "
                         "regime (got dtype %d, %d slices)",
                         dt, sl, y_dtype, y_slices);
    if (T == 0)
        return MOE_OK;
    if (!x_f16 || !perm || !offsets || !d_expert_blobs || !y)
        return set_error(MOE_EINVAL, "moe_expert_ffn_w4a16: null pointer");
    if (((uintptr_t)x_f16 | (uintptr_t)y) & 15u)
        return set_error(MOE_EINVAL, "moe_expert_ffn_w4a16: x and y must be 16-byte aligned");
    if (need && (!ws || ws_bytes < need))
        return set_error(MOE_ENOMEM, "moe_expert_ffn_w4a16: workspace %zu < %zu bytes", ws_bytes,
                         need);
    const int fmt = (regime & MOE_W4_ZERO_POINT) ? MOE_FMT_ZP : MOE_FMT_SYM;
    if (r == MOE_REGIME_DECODE)
        return launch_ffn_decode(x_f16, perm, offsets, d_expert_blobs, nullptr, T, H, I, E, k,
                                 group, fmt, decode_yflags(regime), static_cast<float *>(y),
                                 stream, nullptr);
    if (r == MOE_REGIME_SMALL)
        return launch_ffn_small(x_f16, perm, offsets, d_expert_blobs, T, H, I, E, k, group, fmt, y,
                                ws, stream);
    return launch_ffn_batched(x_f16, perm, offsets, d_expert_blobs, T, H, I, E, k, group, fmt, y,
                              ws, stream);
}

size_t moe_shared_ffn_workspace_bytes(int T, int H, int Is)
{
    return shared_ffn_ws_bytes(T, H, Is);
}

int moe_shared_ffn_f16(const void *x_f16, const void *wg, const void *wu, const void *wd, int T,
                       int H, int Is, float *out_f32, void *ws, size_t ws_bytes,
                       hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    if (T < 0 || H <= 0 || Is <= 0)
        return set_error(MOE_EINVAL, "moe_shared_ffn_f16: bad sizes T=%d H=%d Is=%d", T, H, Is);
    if (!h_supported(H) || Is % 64 || Is > 8192)
        return set_error(MOE_EUNSUPPORTED,
                         "moe_shared_ffn_f16: outside the envelope (H=%d, Is=%d)", H, Is);
    if (T == 0)
        return MOE_OK;
    if (!x_f16 || !wg || !wu || !wd || !out_f32)
        return set_error(MOE_EINVAL, "moe_shared_ffn_f16: null pointer");
    const size_t need = moe_shared_ffn_workspace_bytes(T, H, Is);
    if (!ws || ws_bytes < need)
        return set_error(MOE_ENOMEM, "moe_shared_ffn_f16: workspace %zu < %zu bytes", ws_bytes,
                         need);
    if (T <= SHARED_GEMV_MAX_T)
        return launch_shared_gemv(x_f16, wg, wu, wd, T, H, Is, out_f32, ws, stream);
    return launch_shared_batched(x_f16, wg, wu, wd, T, H, Is, out_f32, ws, stream);
}

static int check_combine_args(const char *fn, const void *y, int y_dtype, int y_slices,
                              const int32_t *inv_perm, const float *topk_w, int T, int H, int k,
                              const void *out_f16)
{
    if (T < 0 || H <= 0 || k <= 0 || k > 16 || y_slices <= 0)
        return set_error(MOE_EINVAL, "%s: bad sizes T=%d H=%d k=%d slices=%d", fn, T, H, k,
                         y_slices);
    if (y_dtype != MOE_DTYPE_F16 && y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_F32_PM)
        return set_error(MOE_EINVAL, "%s: bad y dtype %d", fn, y_dtype);
    if (y_dtype == MOE_DTYPE_F32_PM && H > 0 && H % 8 == 0 && !partial_order_ok(H))
        return set_error(MOE_EINVAL, "%s: H=%d has no partial-major column order", fn, H);
    if (y_dtype == MOE_DTYPE_F16 && y_slices != 1)
        return set_error(MOE_EINVAL, "%s: fp16 y has exactly one slice", fn);
    if (H % 8)
        return set_error(MOE_EUNSUPPORTED, "%s: H=%d must be a multiple of 8", fn, H);
    if (T > 0 && (!y || !topk_w || !out_f16))   // inv_perm NULL: y in token order
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    if (reinterpret_cast<uintptr_t>(y) % 16)
        return set_error(MOE_EINVAL, "%s: y must be 16-byte aligned", fn);
    return MOE_OK;
}

int moe_combine(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                const float *topk_w, const float *shared_f32, const void *residual_f16, int T,
                int H, int k, void *out_f16, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    const int rc = check_combine_args("moe_combine", y, y_dtype, y_slices, inv_perm, topk_w, T,
                                      H, k, out_f16);
    if (rc || T == 0)
        return rc;
    return launch_combine(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32, nullptr, nullptr,
                          residual_f16, T, H, k, out_f16, stream);
}

int moe_combine_gated(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                      const float *topk_w, const float *shared_f32, const void *x_f16,
                      const void *shared_gate_w_f16, const void *residual_f16, int T, int H,
                      int k, void *out_f16, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    const int rc = check_combine_args("moe_combine_gated", y, y_dtype, y_slices, inv_perm,
                                      topk_w, T, H, k, out_f16);
    if (rc || T == 0)
        return rc;
    if (!shared_f32 || !x_f16 || !shared_gate_w_f16)
        return set_error(MOE_EINVAL, "moe_combine_gated: null shared, x or gate pointer");
    if (((uintptr_t)x_f16 | (uintptr_t)shared_gate_w_f16) & 15)
        return set_error(MOE_EINVAL, "moe_combine_gated: x and gate vector need 16-byte alignment");
    return launch_combine(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32, x_f16,
                          shared_gate_w_f16, residual_f16, T, H, k, out_f16, stream);
}

// One decode token of at most 64 experts, fp32 slice partials: the fused
// launch; anything else runs the two calls it stands for.
static bool combine_route_fused(int T, int E, int y_dtype, int y_slices)
{
    return T == 1 && E <= 64 && (y_dtype == MOE_DTYPE_F32 || y_dtype == MOE_DTYPE_F32_PM) &&
           y_slices > 1;
}

size_t moe_combine_route_permute_workspace_bytes(int T, int k_next, int E)
{
    const size_t rp = moe_route_permute_workspace_bytes(T, k_next, E);
    const size_t cr = combine_route_ws_bytes();
    return (T == 1 && E > 0 && E <= 64 && cr > rp) ? cr : rp;
}

int moe_combine_route_permute(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                              const float *topk_w, const float *shared_f32, const void *x_f16,
                              const void *shared_gate_w_f16, const void *residual_f16, int T,
                              int H, int k, void *out_f16, const void *w_router_f16,
                              const float *logit_bias, int E, int k_next, unsigned flags,
                              int32_t *topk_idx, float *topk_w_next, int32_t *counts,
                              int32_t *offsets, int32_t *perm, int32_t *inv_perm_next, void *ws,
                              size_t ws_bytes, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    const char *fn = "moe_combine_route_permute";
    int rc = check_combine_args(fn, y, y_dtype, y_slices, inv_perm, topk_w, T, H, k, out_f16);
    if (rc)
        return rc;
    if (shared_gate_w_f16) {
        if (!shared_f32 || !x_f16)
            return set_error(MOE_EINVAL, "%s: a gate needs the shared output and x", fn);
        if (((uintptr_t)x_f16 | (uintptr_t)shared_gate_w_f16) & 15)
            return set_error(MOE_EINVAL, "%s: x and gate vector need 16-byte alignment", fn);
    }
    rc = check_route_args(fn, out_f16, w_router_f16, T, H, E, k_next, flags, topk_idx,
                          topk_w_next);
    if (rc)
        return rc;
    if (!counts || !offsets || (T > 0 && (!perm || !inv_perm_next)))
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    const size_t need = moe_combine_route_permute_workspace_bytes(T, k_next, E);
    if (need && (!ws || ws_bytes < need))
        return set_error(MOE_ENOMEM, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    if (combine_route_fused(T, E, y_dtype, y_slices))
        return launch_combine_route(static_cast<const float *>(y), y_dtype == MOE_DTYPE_F32_PM,
                                    y_slices, inv_perm, topk_w,
                                    shared_f32, x_f16, shared_gate_w_f16, residual_f16, H, k,
                                    out_f16, w_router_f16, logit_bias, E, k_next, flags, ws,
                                    topk_idx, topk_w_next, counts, offsets, perm, inv_perm_next,
                                    nullptr, stream);
    if (T > 0) {
        rc = launch_combine(y, y_dtype, y_slices, inv_perm, topk_w, shared_f32,
                            shared_gate_w_f16 ? x_f16 : nullptr, shared_gate_w_f16, residual_f16,
                            T, H, k, out_f16, stream);
        if (rc)
            return rc;
    }
    return moe_route_permute(out_f16, w_router_f16, logit_bias, T, H, E, k_next, flags, topk_idx,
                             topk_w_next, counts, offsets, perm, inv_perm_next, ws, ws_bytes,
                             stream);
}

size_t moe_logit_partials_bytes(void) { return (size_t)64 * 64 * sizeof(float); }

int moe_logit_partials(const void *x_f16, const void *w_router_f16, int T, int H, int E,
                       float *logit_partials, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    const char *fn = "moe_logit_partials";
    if (T < 0 || H <= 0 || E <= 0)
        return set_error(MOE_EINVAL, "%s: bad shape T=%d H=%d E=%d", fn, T, H, E);
    if (T != 1 || E > 64)
        return set_error(MOE_EUNSUPPORTED, "%s: one token of at most 64 experts only (T=%d, E=%d)",
                         fn, T, E);
    if (!x_f16 || !w_router_f16 || !logit_partials)
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    if (((uintptr_t)x_f16 | (uintptr_t)w_router_f16) & 15u)
        return set_error(MOE_EINVAL, "%s: x and the router must be 16-byte aligned", fn);
    return launch_logit_partials(x_f16, w_router_f16, H, E, logit_partials, stream);
}

int moe_combine_route_partials(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                               const float *topk_w, const float *shared_f32, const void *x_f16,
                               const void *shared_gate_w_f16, const void *residual_f16, int T,
                               int H, int k, void *out_f16, const void *w_router_f16, int E,
                               float *logit_partials, hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    const char *fn = "moe_combine_route_partials";
    int rc = check_combine_args(fn, y, y_dtype, y_slices, inv_perm, topk_w, T, H, k, out_f16);
    if (rc)
        return rc;
    if (shared_gate_w_f16) {
        if (!shared_f32 || !x_f16)
            return set_error(MOE_EINVAL, "%s: a gate needs the shared output and x", fn);
        if (((uintptr_t)x_f16 | (uintptr_t)shared_gate_w_f16) & 15)
            return set_error(MOE_EINVAL, "%s: x and gate vector need 16-byte alignment", fn);
    }
    if (!w_router_f16 || !logit_partials)
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    if (E <= 0 || E > 64 || T != 1 || !combine_route_fused(T, E, y_dtype, y_slices))
        return set_error(MOE_EUNSUPPORTED,
                         "%s: one decode token of at most 64 experts only (T=%d, E=%d)", fn, T,
                         E);
    return launch_combine_route(static_cast<const float *>(y), y_dtype == MOE_DTYPE_F32_PM,
                                y_slices, inv_perm, topk_w, shared_f32, x_f16, shared_gate_w_f16,
                                residual_f16, H, k, out_f16, w_router_f16, nullptr, E, k, 0u,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                logit_partials, stream);
}

int moe_expert_ffn_w4a16_routed(const void *x_f16, const float *logit_partials,
                                const float *logit_bias, int E, int k, unsigned flags,
                                int32_t *topk_idx, float *topk_w, int32_t *counts,
                                int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                                const void *const *d_expert_blobs, int T, int H, int I,
                                int group, int regime, void *y, int y_dtype, int y_slices,
                                hipStream_t stream)
{
    MOE_API_RANGE();
    clear_error();
    const char *fn = "moe_expert_ffn_w4a16_routed";
    if (flags & ~(unsigned)MOE_RENORM)
        return set_error(MOE_EINVAL, "%s: unknown flags 0x%x", fn, flags);
    int r = 0, dt = 0, sl = 0;
    size_t need = 0;
    int rc = moe_expert_ffn_plan(T, H, I, E, k, group, regime, &r, &dt, &sl, &need);
    if (rc)
        return rc;
    if (T != 1 || E > 64 || r != MOE_REGIME_DECODE || need != 0)
        return set_error(MOE_EUNSUPPORTED,
                         "%s: one decode token of at most 64 experts only (T=%d, E=%d)", fn, T,
                         E);
    if (y_dtype != dt || y_slices != sl)
        return set_error(MOE_EINVAL,
                         "%s: y must be dtype %d with %d slices for this regime (got dtype %d, "
                         "%d slices)",
                         fn, dt, sl, y_dtype, y_slices);
    if (!x_f16 || !logit_partials || !topk_idx || !topk_w || !counts || !offsets || !perm ||
        !inv_perm || !d_expert_blobs || !y)
        return set_error(MOE_EINVAL, "%s: null pointer", fn);
    if (((uintptr_t)x_f16 | (uintptr_t)y) & 15u)
        return set_error(MOE_EINVAL, "%s: x and y must be 16-byte aligned", fn);
    const DecodeRoute rt{logit_partials, logit_bias, flags, topk_idx, counts, offsets, perm,
                         inv_perm, topk_w};
    const int fmt = (regime & MOE_W4_ZERO_POINT) ? MOE_FMT_ZP : MOE_FMT_SYM;
    return launch_ffn_decode(x_f16, nullptr, nullptr, d_expert_blobs, nullptr, T, H, I, E, k,
                             group, fmt, decode_yflags(regime), static_cast<float *>(y), stream,
                             &rt);
}

}  // extern "C"
