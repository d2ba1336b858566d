/*
 * moe_w4a16.h -- C ABI of libmoe_w4a16.so, the MI355X (gfx950) hot path of a
 * sparsely-activated Mixture-of-Experts layer with INT4 weight-only routed
 * experts and FP16 activations (W4A16).
 *
 * Sources.  The pages describe the method, not an API:
 *  - Horizon RunMap, "Prévia Técnica" (horizonrunmap.com/pt):
 *    "02 / A solução", "03 / Arquitetura" -- the router chooses experts; own
 *    kernels combine compact INT4 weights and FP16 scales with FP16
 *    activations and hand the result back to the model, never keeping an
 *    expanded expert; non-routed parts stay FP16; the optional slot cache
 *    (resident-qpacked-cache-v1) with an immutable host source, temporary
 *    slots, generation publish and consumer retirement.
 *    "08 / Comportamento do modelo" -- W4 = INT4 expert weights with FP16
 *    scales, A16 = FP16 activations, FP32 accumulation stages with explicit
 *    roundings.
 *  - Hamidun News, "Desenvolvedor do Strata cria mapa ao vivo de 24 576
 *    especialistas MoE em uma GTX 1070", "Como 125 bilhões de parâmetros
 *    cabem em 8 GB" -- hot experts resident, the rest loaded on demand,
 *    eviction by an access counter with decay.
 * Where the pages are silent (softmax form, tie-break, SwiGLU, group size,
 * quantiser rounding, logit summation order, eviction constants) the
 * functions follow fixed readings stated next to each declaration.
 *
 * Conventions
 *  - Every function returns MOE_OK (0) or a negative MOE_E* code; a
 *    thread-local message is available from moe_last_error().  No exception
 *    crosses the ABI.
 *  - Shapes and pointers are validated on the host before anything is
 *    launched; on error nothing is launched and outputs are untouched.
 *  - "device" pointers are HIP device memory (hipMalloc / torch CUDA
 *    tensors) of the current device; "host" pointers are CPU memory.
 *  - The caller allocates and owns every activation, weight, output and
 *    workspace; compute calls never allocate.  The slot pool owns its HBM
 *    slots, tables, side stream and events (allocated once at creation).
 *  - Compute calls are asynchronous on the caller's stream and do not
 *    synchronise with the host.  Inputs must be finite (not checked).
 *  - Layouts are row-major; fp16 is IEEE binary16; int32 indices.
 *
 * Kernel envelope (MOE_EUNSUPPORTED outside it): H in {256, 512, 1024, 2048};
 * I a multiple of 64 (up to 8192); group g in {32, 64, 128} dividing
 * H and I; E <= 1024; k <= 16 and k <= E; T*k < 2^31.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ codes */
enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null pointer, bad size, k > E, g does not divide H/I ... */
    MOE_EUNSUPPORTED = -2,  /* valid but outside the kernel envelope */
    MOE_ENOMEM = -3,        /* workspace too small, or pool allocation failed */
    MOE_EHIP = -4,          /* a HIP runtime call failed (message has the hipError_t) */
    MOE_ECAPACITY = -5,     /* the slot pool rejects the profile or the routed set */
    MOE_ESTATE = -6         /* slot pool used out of order */
};

enum { MOE_RENORM = 1u };                       /* moe_route flag */
enum { MOE_REGIME_AUTO = 0, MOE_REGIME_DECODE = 1, MOE_REGIME_BATCHED = 2, MOE_REGIME_SMALL = 3 };
/* OR'd into the regime of moe_expert_ffn_plan / moe_expert_ffn_w4a16: y rows
 * in token order (row t*k + j) instead of sorted order; see below. */
enum { MOE_Y_TOKEN_ORDER = 0x100 };
/* OR'd into the same regime: the DECODE partials' columns in partial-major
 * order (the plan then reports MOE_DTYPE_F32_PM).  With C = H/8 chunks of 8
 * columns and q = ceil(C/64), column c of chunk u = 64m + j (j < 64) is stored
 * at column 8(jq + m) + c mod 8: the chunks j, j+64, ... that form partial j
 * of the router's pinned logit sum lie side by side, so a reader that owns
 * partial j reads whole lines.  Needs C <= 64 or C a multiple of 64. */
enum { MOE_Y_PARTIAL_ORDER = 0x400 };
/* y dtypes: fp16, fp32 (decode slices), fp32 in partial-major column order. */
enum { MOE_DTYPE_F16 = 0, MOE_DTYPE_F32 = 1, MOE_DTYPE_F32_PM = 2 };
/* Expert blob formats: symmetric codes, or codes with a zero point per group
 * (lucashiago.com.br explainer, step 1: each block carries a scale and a zero
 * point).  MOE_W4_ZERO_POINT is OR'd into the regime of moe_expert_ffn_plan /
 * moe_expert_ffn_w4a16 / moe_pool_layer_args when the blobs are FMT_ZP. */
enum { MOE_FMT_SYM = 0, MOE_FMT_ZP = 1 };
enum { MOE_W4_ZERO_POINT = 0x200 };

/* Thread-local text of the last error on this thread ("" if none). */
const char *moe_last_error(void);

/*
 * Zero-fills ws_bytes bytes of a device workspace with a kernel on `stream`
 * (no hipMemsetAsync, so it may be recorded in a captured graph).  It is the
 * initial fill that moe_route_permute and moe_shared_ffn_f16 require, and the
 * way back after a call that did not run to completion (a failed launch, an
 * aborted graph replay): those calls keep an arrival ticket / arrival counters
 * at the start of their workspace, every completed call leaves them zero, and
 * a non-zero leftover would make the next call skip its final reduction.
 * Any address and size; MOE_EINVAL for a null ws with ws_bytes > 0.
 */
int moe_workspace_clear(void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------- expert blob */
/*
 * Canonical expert blob (Horizon RunMap "02 / A solução": compact weights
 * and FP16 scales in separate formats; lucashiago.com.br explainer step 1:
 * every block of weights carries its scale).  Six sections, each 256-byte
 * aligned:  gate_q[I][H/2], up_q[I][H/2], down_q[H][I/2]  (u8: element 2b in
 * the low nibble of byte b, element 2b+1 in the high nibble, stored as
 * u = q + 8 with q in [-7, 7]) then gate_s[I][H/g], up_s[I][H/g],
 * down_s[H][I/g] (fp16 scales, one per group of g along the input dim).
 * W = q * s.  offsets[6] get the section offsets, *total_bytes the blob size.
 * Host-only, no GPU needed.  MOE_EINVAL on bad sizes.
 */
int moe_blob_layout(int H, int I, int group, int64_t offsets[6], int64_t *total_bytes);

/*
 * Quantise n experts to canonical blobs on the device (symmetric group-wise
 * INT4; reading: s = fp16_rne(fp32(amax/7)), q = clamp(rne(fp32(w/s)), -7, 7),
 * q = 0 when s = 0).
 *   wg, wu: device fp32 [n][I][H]; wd: device fp32 [n][H][I] (row-major)
 *   blobs:  device, n consecutive blobs of total_bytes each (output)
 * Offline step (load time), not part of the per-token path.
 */
int moe_quantize_experts(const float *wg, const float *wu, const float *wd,
                         int n, int H, int I, int group, void *blobs, hipStream_t stream);

/*
 * Byte bijection from canonical blobs to the device layout the kernels read
 * (same size; never expands to fp16).  Applied once at load, to resident
 * weights and to the pinned source of the slot pool.
 *   src: device, n canonical blobs; dst: device, n blobs (must not overlap src)
 * Device layout: gate and up rows fused into 64-row blocks (32 gate rows then
 * the 32 up rows of the same intermediate indices), down in 64-row blocks;
 * inside a block, 32-element input chunks of all 64 rows are contiguous
 * (16 bytes per row: four dwords holding elements 0-7, 16-23, 8-15, 24-31,
 * each with element 2i at bits 4i and element 2i+1 at bits 16+4i, so that
 * a nibble pair converts in registers with one mask);
 * scales in [block][group][64 rows] order.
 */
int moe_prepack_experts(const void *src, int n, int H, int I, int group, void *dst,
                        hipStream_t stream);

/* Inverse of moe_prepack_experts (for inspection and tests). */
int moe_unpack_experts(const void *src, int n, int H, int I, int group, void *dst,
                       hipStream_t stream);

/*
 * Zero-point (asymmetric) INT4 blobs (lucashiago.com.br explainer, step 1:
 * each block of weights carries a scale and a zero point).  Canonical blob:
 * the six sections above at the same offsets, then gate_z[I][H/g],
 * up_z[I][H/g], down_z[H][I/g] (u8, one zero point z in [0, 15] per group),
 * each 256-byte aligned; a stored nibble u in [0, 15] means W = (u - z) * s.
 * (MOE_FMT_SYM is the case z = 8 with no zero-point sections.)
 * moe_blob_layout_fmt: offsets[0..8] (the last three 0 for MOE_FMT_SYM).
 * moe_quantize_experts_fmt with MOE_FMT_ZP quantises per group with the
 * reading lo = min(min w, 0), hi = max(max w, 0), s = fp16_rne((hi - lo)/15),
 * z = clamp(rne(-lo/s), 0, 15), u = clamp(rne(w/s) + z, 0, 15), quotients in
 * fp32; s = 0 gives z = u = 0.  moe_prepack_experts_fmt /
 * moe_unpack_experts_fmt: the device layout of moe_prepack_experts plus the
 * zero points in the scales' order (one byte each) after the scales.  The
 * expert kernels read such blobs when MOE_W4_ZERO_POINT is OR'd into the
 * regime.  MOE_EINVAL for an unknown fmt, else as the symmetric calls.
 */
int moe_blob_layout_fmt(int H, int I, int group, int fmt, int64_t offsets[9],
                        int64_t *total_bytes);
int moe_quantize_experts_fmt(const float *wg, const float *wu, const float *wd, int n, int H,
                             int I, int group, int fmt, void *blobs, hipStream_t stream);
int moe_prepack_experts_fmt(const void *src, int n, int H, int I, int group, int fmt, void *dst,
                            hipStream_t stream);
int moe_unpack_experts_fmt(const void *src, int n, int H, int I, int group, int fmt, void *dst,
                           hipStream_t stream);

/*
 * The same bijection on the host, one blob (src and dst host memory of the
 * canonical blob size, not overlapping): for a source that lives in host
 * memory, such as the pinned INT4 source of the slot pool, so that loading it
 * needs no device round trip.  Bytes identical to moe_prepack_experts_fmt /
 * moe_unpack_experts_fmt.  No GPU needed.  MOE_EINVAL on bad arguments.
 */
int moe_prepack_expert_host(const void *src, int H, int I, int group, int fmt, void *dst);
int moe_unpack_expert_host(const void *src, int H, int I, int group, int fmt, void *dst);

/* ------------------------------------------------------------ router */
/*
 * Router softmax + top-k (Horizon RunMap "03 / Arquitetura": the router
 * selects the experts of each token; routing stays outside INT4, "08").
 *   x_f16:        device fp16 [T][H] activations
 *   w_router_f16: device fp16 [E][H]
 *   logit_bias:   device fp32 [E] added to every logit after the dot product,
 *                 or NULL
 *   flags:        MOE_RENORM renormalises the k weights to sum to one
 *   topk_idx:     device int32 [T][k] (output), experts by (logit desc,
 *                 index asc) -- ties go to the lower expert index
 *   topk_w:       device fp32 [T][k] (output), softmax over all E logits at
 *                 the chosen experts
 *   ws:           device scratch of moe_route_workspace_bytes(T, E) bytes
 *                 (0 for T <= 8, where ws may be NULL; above that it holds the
 *                 T x E fp32 logits between the logit and top-k launches;
 *                 contents need no initialisation); MOE_ENOMEM if too small
 * Logits are fp32 in a fixed summation order (chunks of 8 elements of H go
 * to partial (chunk mod 64) in increasing order, partials combined by an xor
 * butterfly 32,16,8,4,2,1), so the indices are reproducible bit for bit.
 * T = 0 is a no-op.
 */
size_t moe_route_workspace_bytes(int T, int E);
int moe_route(const void *x_f16, const void *w_router_f16, const float *logit_bias,
              int T, int H, int E, int k, unsigned flags,
              int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
              hipStream_t stream);

/* ------------------------------------------------------- permutation */
/*
 * Token-to-expert grouping (the pages' grouped executor computes experts in
 * groups, Horizon RunMap "04 / Resultados").  Stable counting sort of the
 * flat index f = t*k + j by expert topk_idx[f]:
 *   counts   device int32 [E]     tokens routed to each expert
 *   offsets  device int32 [E+1]   exclusive scan of counts, offsets[E] = T*k
 *   perm     device int32 [T*k]   sorted position -> f (f ascending per expert)
 *   inv_perm device int32 [T*k]   f -> sorted position
 * ws: device scratch of at least moe_permute_workspace_bytes(T, k, E) bytes
 * (contents need no initialisation).  Bit-exact: one correct answer.
 */
size_t moe_permute_workspace_bytes(int T, int k, int E);
int moe_permute(const int32_t *topk_idx, int T, int k, int E,
                int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_route followed by moe_permute, with the same arguments and results
 * (same passages and readings).  For small T (T <= 5 with E <= 128, T <= 4
 * with E > 128, where one selecting workgroup still beats two launches) both
 * run in one launch: the logits are spread over many workgroups, and the
 * workgroup that finishes last (an atomic ticket in ws; no workgroup ever
 * waits for another) does the top-k, the softmax and the stable sort -- the
 * decode path's one launch instead of two.  For larger T it runs moe_route's
 * launches (logits into ws, then top-k) followed by moe_permute's, on the
 * same ws.
 * ws: device scratch of moe_route_permute_workspace_bytes(T, k, E) bytes.  It
 * must be zero-filled before its first use by this function; every completed
 * call leaves it reusable (the ticket, its first 256 bytes, back at zero),
 * for any T.  Calls that share one workspace must not run concurrently.
 */
size_t moe_route_permute_workspace_bytes(int T, int k, int E);
int moe_route_permute(const void *x_f16, const void *w_router_f16, const float *logit_bias,
                      int T, int H, int E, int k, unsigned flags,
                      int32_t *topk_idx, float *topk_w, int32_t *counts, int32_t *offsets,
                      int32_t *perm, int32_t *inv_perm, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * moe_route_permute without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (minus ws), results and
 * errors as moe_route_permute; it calls no hipMalloc/hipFree and no
 * allocating routine.  Its workspace is a 16 MiB array inside the library, one
 * per GPU, held until the process ends; on the first call on a device its
 * ticket is cleared by a kernel on `stream`, and every completed call leaves
 * it clear again.  Shapes whose workspace (moe_route_permute_workspace_bytes)
 * exceeds 16 MiB are rejected with MOE_ENOMEM before anything is launched
 * (T = 4096 tokens with E = 512 experts and k = 10 need 8.7 MB; the
 * workspace grows as 4*T*E bytes).  Every call on one GPU shares that
 * array: calls that overlap in time on one GPU (different streams, or
 * threads) race and must not be made.
 */
int moe_route_permute_noalloc(const void *x_f16, const void *w_router_f16,
                              const float *logit_bias, int T, int H, int E, int k, unsigned flags,
                              int32_t *topk_idx, float *topk_w, int32_t *counts, int32_t *offsets,
                              int32_t *perm, int32_t *inv_perm, hipStream_t stream);

/* ------------------------------------------------ routed expert FFN */
/*
 * What moe_expert_ffn_w4a16 will do for a shape: the resolved regime, the
 * dtype and number of slices of y, and the workspace it needs.  Host-only.
 * AUTO picks DECODE for T <= 4 tokens, SMALL for T <= 32, else BATCHED.
 *   DECODE : one launch, rows of an expert one after another on the vector
 *            ALUs.  y is fp32 [slices][T*k][H], partial sums over
 *            intermediate slices of 32 (slices = I/32); moe_combine adds them.
 *   SMALL  : T <= 32 (Horizon RunMap "10 / Próximas perguntas": concurrent
 *            use).  Each expert's weights are streamed once and its <= T rows
 *            multiplied on the matrix cores; gate/up then down, h in ws.
 *            T > 32 is MOE_EUNSUPPORTED.  y is fp16 [1][T*k][H].
 *   BATCHED: tiled grouped GEMM, any T.  y is fp16 [1][T*k][H].
 * regime may carry MOE_Y_TOKEN_ORDER and MOE_Y_PARTIAL_ORDER (DECODE only:
 * MOE_EUNSUPPORTED when the resolved regime is another; with the second, y_dtype
 * is MOE_DTYPE_F32_PM) and MOE_W4_ZERO_POINT (any regime: the blobs are
 * MOE_FMT_ZP); resolved_regime is returned without them.
 */
int moe_expert_ffn_plan(int T, int H, int I, int E, int k, int group, int regime,
                        int *resolved_regime, int *y_dtype, int *y_slices,
                        size_t *ws_bytes);

/*
 * Routed-expert SwiGLU FFN computed directly from INT4 weights
 * (Horizon RunMap "03 / Arquitetura" and "08": the kernel reads compact
 * weights and FP16 scales, converts what it needs during the computation,
 * uses FP16 activations and FP32 accumulation, and never keeps an expanded
 * expert).  For each sorted row p of expert e and token t = perm[p] / k:
 *   h = silu(Wg[e] x_t) * (Wu[e] x_t),   y_p = Wd[e] h,   W = q * s.
 *   x_f16          device fp16 [T][H]; 16-byte aligned
 *   perm, offsets  device, from moe_permute
 *   d_expert_blobs device array of E device pointers to prepacked blobs
 *                  (moe_prepack_experts); an entry may be NULL only for an
 *                  expert no token routes to, except in the DECODE regime,
 *                  where a routed expert with a NULL entry is skipped (its y
 *                  rows are left unwritten for another launch to fill)
 *   y              device output, layout from moe_expert_ffn_plan, 16-byte
 *                  aligned; y_dtype and y_slices must equal the plan's
 *                  (MOE_EINVAL otherwise).
 *                  Row p holds sorted row p; with MOE_Y_TOKEN_ORDER in regime
 *                  (DECODE only) the result of sorted row p goes to row
 *                  perm[p] = t*k + j instead, so that moe_combine needs no
 *                  inv_perm (one dependent memory round trip less); with
 *                  MOE_Y_PARTIAL_ORDER each row's columns are stored in
 *                  partial-major order (MOE_DTYPE_F32_PM)
 *   ws             device scratch of the plan's size (may be NULL if 0)
 * Rounding: DECODE converts h to fp16 before the down projection; SMALL and
 * BATCHED convert the weights to fp16(q * s) and store h and y as fp16.
 * Everything else accumulates in fp32.
 */
int moe_expert_ffn_w4a16(const void *x_f16, const int32_t *perm, const int32_t *offsets,
                         const void *const *d_expert_blobs,
                         int T, int H, int I, int E, int k, int group, int regime,
                         void *y, int y_dtype, int y_slices,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------ shared FP16 expert */
/*
 * Separate FP16 non-routed expert (Horizon RunMap "03": parts outside the
 * routed experts stay FP16).  SwiGLU FFN applied to every token:
 *   s_t = Wd (silu(Wg x_t) * (Wu x_t)),
 *   wg, wu: device fp16 [Is][H];  wd: device fp16 [H][Is]  (row-major)
 *   out_f32: device fp32 [T][H]
 *   ws:      device scratch of moe_shared_ffn_workspace_bytes(T, H, Is) bytes,
 *            zero-filled by the caller before its first use.  Its first 2 KB
 *            hold arrival counters of the split-K reduction; every call
 *            leaves them zero again, so one zero-fill serves any number of
 *            calls (and graph replays) with any T.  Calls that share a
 *            workspace must not overlap.
 * h is rounded to fp16 between the projections; fp32 accumulation.  The
 * order of the fp32 additions depends on T, H and Is only, so repeated calls
 * give identical bits.
 */
size_t moe_shared_ffn_workspace_bytes(int T, int H, int Is);
int moe_shared_ffn_f16(const void *x_f16, const void *wg, const void *wu, const void *wd,
                       int T, int H, int Is, float *out_f32,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ combine */
/*
 * Router-weighted combine (Horizon RunMap "03": results go back to the rest
 * of the model).  For each token t and column c:
 *   out[t,c] = fp16_rne( r + sum_j w[t,j] * Y(inv_perm[t*k+j], c) + s[t,c] )
 * where Y(p,c) is y[p,c] (y_dtype F16, y_slices 1) or the sum over slices of
 * y[slice][p][c] (F32; the slices summed in two contiguous halves, each in
 * slice order, then the halves added; F32_PM: the same with column c read
 * from its partial-major position), r = residual[t,c] or 0, s the
 * shared-expert output or 0.  fp32 sum in the order: experts j = 0..k-1
 * (each the slice sum), shared, residual; one final rounding.
 *   y            device, from moe_expert_ffn_w4a16; 16-byte aligned
 *   inv_perm     device int32 [T*k], or NULL when y is in token order
 *                (MOE_Y_TOKEN_ORDER): then Y(t*k+j, c) is read directly
 *   topk_w       device fp32 [T][k]
 *   shared_f32   device fp32 [T][H] or NULL
 *   residual_f16 device fp16 [T][H] or NULL (may alias out_f16)
 *   out_f16      device fp16 [T][H]
 * Errors: MOE_EINVAL for bad sizes or dtype (k outside 1..16, F16 y with
 * more than one slice, F32_PM with an H that has no partial-major order), a
 * null y/topk_w/out pointer or a misaligned y; MOE_EUNSUPPORTED when H is
 * not a multiple of 8.
 */
int moe_combine(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                const float *topk_w, const float *shared_f32, const void *residual_f16,
                int T, int H, int k, void *out_f16, hipStream_t stream);

/*
 * Combine with a gated shared expert.  The pages run a second model family
 * with 60 routed experts per layer and a top-4 executor (Horizon RunMap
 * technical preview, residency results table, top4-fused-v1 rows) without
 * printing its layer; in that family the shared expert's output is scaled per
 * token by a sigmoid of one more linear function of the token (a reading; no
 * bias term).  Same as moe_combine except that the shared term is
 *   G_t * s[t,c],   G_t = 1 / (1 + exp(-sum_c x[t,c] * wsg[c])),
 * the dot taken in fp32 (any order; G_t is not a discrete decision).
 *   shared_f32         device fp32 [T][H], required
 *   x_f16              device fp16 [T][H], the layer input; 16-byte aligned
 *   shared_gate_w_f16  device fp16 [H]; 16-byte aligned
 * Errors: MOE_EINVAL for a null shared/x/gate pointer or misalignment, else
 * as moe_combine.
 */
int moe_combine_gated(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                      const float *topk_w, const float *shared_f32, const void *x_f16,
                      const void *shared_gate_w_f16, const void *residual_f16, int T, int H,
                      int k, void *out_f16, hipStream_t stream);

/*
 * Combine of one layer fused with route + permute of the next (Horizon
 * RunMap "03 / Arquitetura": the experts' results return to the model, whose
 * next layer's router then selects its experts; the pages run 16 such layers
 * per token).  Exactly the two calls it stands for, bit for bit:
 *   moe_combine (shared_gate_w_f16 NULL) or moe_combine_gated (non-NULL:
 *     then shared_f32 and x_f16, the layer's input, are required) with y,
 *     y_dtype, y_slices, inv_perm, topk_w, shared_f32, residual_f16, T, H, k,
 *     writing out_f16;
 *   then moe_route_permute(out_f16, w_router_f16, logit_bias, T, H, E, k_next,
 *     flags, topk_idx, topk_w_next, counts, offsets, perm, inv_perm_next).
 * One launch when T = 1, E <= 64 and y holds fp32 slices (y_slices > 1, the
 * decode layout; with MOE_DTYPE_F32_PM every block of that launch reads whole
 * lines); otherwise the two calls run in turn on `stream`.
 *   ws  device workspace of moe_combine_route_permute_workspace_bytes(T,
 *       k_next, E) bytes, zero-filled before the first call
 *       (moe_workspace_clear).  The fused launch leaves its first 256 bytes
 *       alone and passes the next layer's logit partials from block to block
 *       through tagged words after them (the selecting block polls them; no
 *       other block waits), with a call counter at the end; so the same
 *       workspace may also serve moe_route_permute, whose ticket lives in the
 *       first 256 bytes.
 * The layer's routing arrays (topk_w, inv_perm) and the next layer's
 * (topk_w_next, inv_perm_next) may be the same arrays: every read of the
 * former precedes every write of the latter.  out_f16 may alias residual_f16
 * but not x_f16.  Errors: those of the two calls, checked before any launch;
 * MOE_ENOMEM for a short workspace.
 */
size_t moe_combine_route_permute_workspace_bytes(int T, int k_next, int E);
int moe_combine_route_permute(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                              const float *topk_w, const float *shared_f32, const void *x_f16,
                              const void *shared_gate_w_f16, const void *residual_f16, int T,
                              int H, int k, void *out_f16, const void *w_router_f16,
                              const float *logit_bias, int E, int k_next, unsigned flags,
                              int32_t *topk_idx, float *topk_w_next, int32_t *counts,
                              int32_t *offsets, int32_t *perm, int32_t *inv_perm_next, void *ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * The same two stacked decode layers split differently: the combine of
 * layer l and only the next layer's logit partials in one launch, then the
 * next layer's routing done inside its expert FFN.  Every workgroup of the
 * FFN folds the partials in the pinned order and selects for itself, so no
 * workgroup waits for another and the combine's launch ends once its
 * partials are stored.  Together the two calls give, bit for bit, what
 * moe_combine_route_permute followed by moe_expert_ffn_w4a16 give (the same
 * out_f16, routing arrays and y).  For one decode token of at most 64 experts
 * (T = 1, E <= 64, y of the decode regime: MOE_DTYPE_F32 or MOE_DTYPE_F32_PM
 * with y_slices > 1); other shapes are MOE_EUNSUPPORTED (use the calls above).
 *
 * moe_combine_route_partials: arguments as moe_combine_route_permute up to
 * logit_bias-less w_router_f16 and E; writes out_f16 and
 *   logit_partials  device fp32 [64][64] (moe_logit_partials_bytes()):
 *                   partial j of expert e's logit at j * 64 + e, partial j
 *                   summing the 8-column chunks j, j + 64, ... of out_f16 in
 *                   the pinned order (Horizon RunMap "08": routing in FP32
 *                   with explicit roundings); rows j >= min(64, H / 8) are not
 *                   written and count as zero.
 * moe_expert_ffn_w4a16_routed: x_f16 (the combine's out_f16), the partials,
 * logit_bias (may be NULL), E, k, flags as moe_route; writes the routing
 * arrays of moe_route_permute (topk_idx, topk_w, counts, offsets, perm,
 * inv_perm) and y as moe_expert_ffn_w4a16 in the DECODE regime (regime may
 * carry MOE_Y_TOKEN_ORDER, MOE_Y_PARTIAL_ORDER and MOE_W4_ZERO_POINT;
 * d_expert_blobs must hold every expert).  Errors: MOE_EINVAL / ENOMEM /
 * EUNSUPPORTED as the calls they replace, checked before any launch.
 * moe_logit_partials: the same partials straight from an fp16 input row
 * that no combine forms (the first layer of a stack): x_f16 device fp16 [H]
 * (T = 1), w_router_f16 device fp16 [E][H] (both 16-byte aligned), into
 * logit_partials as above; routing from them equals moe_route_permute of
 * x_f16 bit for bit.  One launch of min(64, H / 8) one-wave workgroups.
 * Errors: MOE_EINVAL (shape, null, alignment), MOE_EUNSUPPORTED (T != 1,
 * E > 64, H not instantiated), before any launch.
 */
size_t moe_logit_partials_bytes(void);
int moe_logit_partials(const void *x_f16, const void *w_router_f16, int T, int H, int E,
                       float *logit_partials, hipStream_t stream);
int moe_combine_route_partials(const void *y, int y_dtype, int y_slices, const int32_t *inv_perm,
                               const float *topk_w, const float *shared_f32, const void *x_f16,
                               const void *shared_gate_w_f16, const void *residual_f16, int T,
                               int H, int k, void *out_f16, const void *w_router_f16, int E,
                               float *logit_partials, hipStream_t stream);
int moe_expert_ffn_w4a16_routed(const void *x_f16, const float *logit_partials,
                                const float *logit_bias, int E, int k, unsigned flags,
                                int32_t *topk_idx, float *topk_w, int32_t *counts,
                                int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                                const void *const *d_expert_blobs, int T, int H, int I,
                                int group, int regime, void *y, int y_dtype, int y_slices,
                                hipStream_t stream);

/* ------------------------------------------------- expert slot pool */
/*
 * Partial residency (Horizon RunMap "03 / Arquitetura",
 * resident-qpacked-cache-v1; "07 / De volta à oficina": hit, miss, discard):
 * the complete INT4 source stays immutable in pinned host memory; each layer
 * owns C resident slots plus S spare slots in HBM; a miss is copied into a
 * spare slot on a side stream while readers keep the previous generation;
 * once the routed group's copies complete, a new complete generation of the
 * layer's expert table is published; an evicted slot is reused only after
 * the kernels that read it have retired.  Capacity is fixed at creation.
 * Eviction (Strata, decayed access counter; reading): per routed event of a
 * layer, every counter of the layer decays c <- c - (c >> decay_shift)
 * (decay_shift < 0: no decay), routed experts add 65536, hits then misses
 * are touched in ascending id on a use clock, and each miss (ascending id)
 * evicts the resident non-routed expert with the lowest (counter, last use,
 * id).  decay_shift = 0 is plain LRU.  Initial placement: experts 0..C-1.
 */
typedef struct moe_pool *moe_pool_t;

typedef struct {
    int layers;            /* L */
    int experts;           /* E per layer */
    int topk;              /* k */
    int capacity;          /* C resident slots per layer, k <= C <= E */
    int spares;            /* S spare slots per layer, S >= k */
    int decay_shift;       /* counter decay; < 0 disables decay */
    int64_t expert_bytes;  /* bytes of one prepacked blob */
} moe_pool_config;

typedef struct {
    int64_t hits, misses, evictions, h2d_bytes, generation;
} moe_pool_stats_t;

/*
 * pinned_src: host array of L*E host pointers (index l*E + e), each a blob
 * in device layout inside pinned host memory (hipHostMalloc); read-only.
 * Allocates L*(C+S) slots and 2*L tables of E device pointers on the
 * current device, a side stream and events, and uploads the initial
 * placement (synchronously).  MOE_ECAPACITY if C < k, C > E, S < k, or the
 * slots do not fit in free device memory; MOE_EINVAL on bad arguments.
 */
int moe_pool_create(const moe_pool_config *cfg, const void *const *pinned_src,
                    moe_pool_t *out);

/*
 * Make the distinct experts among host_ids[0..n) (the layer's routed ids,
 * copied to the host) resident and publish the layer's next generation.
 * Misses are copied H2D on the side stream into spare slots (waiting for the
 * retirement of earlier readers of those slots); the compute stream is made
 * to wait for the copies and the table update (a call whose experts are all
 * resident republishes the current table: nothing copied, nothing awaited).
 * *d_table_out receives the
 * device array of E blob pointers to pass to moe_expert_ffn_w4a16 on
 * `compute` (NULL for non-resident experts).  `step` (may be NULL) gets this
 * call's counters (hits/misses/evictions/h2d_bytes; generation = new one).
 * MOE_ECAPACITY if the routed set has more misses than spares or more
 * distinct experts than C; MOE_ESTATE if the layer's previous generation was
 * not retired.  On any error the previous generation and all counters are
 * unchanged.
 */
int moe_pool_prepare(moe_pool_t pool, int layer, const int32_t *host_ids, int n,
                     hipStream_t compute, const void *const **d_table_out,
                     moe_pool_stats_t *step);

/*
 * Profile-pinned policy for one layer (local-inference explainer,
 * lucashiago.com.br, step 4: besides keeping what was used last, one can
 * measure usage first and fix the most used experts; such a profile ages when
 * the workload changes).  experts[0..n): host int32, n must equal C, distinct
 * ids in [0, E) -- typically the C most frequent experts of a measured
 * profile.  They are copied into the layer's C resident slots (synchronously;
 * the call waits for the device) and stay there: from now on a routed expert
 * of the set is a hit, and every other routed expert is a miss copied into a
 * spare slot for that generation only, dropped at the layer's next prepare
 * (paid again at its next use; nothing is evicted, evictions stay 0).
 * moe_pool_reset() returns every layer to the decayed-counter policy and the
 * canonical placement.  MOE_EINVAL on bad ids or n != C; MOE_ESTATE if the
 * layer's last generation was not retired.
 */
int moe_pool_pin(moe_pool_t pool, int layer, const int32_t *experts, int n);

/* Record that every kernel enqueued on `compute` so far that reads the
 * layer's current generation has been issued; slots evicted by it become
 * reusable once those kernels finish.  MOE_ESTATE if nothing to retire. */
int moe_pool_retire(moe_pool_t pool, int layer, hipStream_t compute);

/*
 * One pooled MoE layer for a small batch -- the decode loop of a partially
 * resident model -- in one host call, with the same readings as the calls it
 * chains: moe_route_permute on `stream`; the T*k routed ids copied into
 * host_ids (pinned host memory) and waited for (this call blocks the calling
 * thread until they arrive; for one token of at most 64 experts the routing
 * kernel itself writes them, then a sequence flag, into the pool's own
 * coherent pinned buffer and the thread spins on the flag, MOE_EHIP after
 * 10 s, instead of a device-to-host copy and an event wait); moe_pool_prepare
 * on this layer; the routed
 * expert FFN (moe_expert_ffn_w4a16 with the published table and `regime`);
 * moe_pool_retire; moe_combine into out_f16.  E is the pool's expert count.
 * When the routed set has both hits and misses and the decode kernel runs,
 * the hits are computed first, on the previous generation's table (where
 * every hit already sits in its slot and no miss appears), while the misses
 * are copied; a second launch on the new table then computes the misses.
 * Every buffer is the caller's, sized as for those calls (route_ws:
 * moe_route_permute_workspace_bytes, zero-filled before its first use;
 * y / ffn_ws: moe_expert_ffn_plan).  Errors are those of the chained calls;
 * the first one stops the chain (a failure in prepare leaves the layer's
 * previous generation published).
 */
typedef struct {
    const void *x_f16;          /* device fp16 [T][H] */
    const void *w_router_f16;   /* device fp16 [E][H] */
    const float *logit_bias;    /* device fp32 [E] or NULL */
    int T, H, I, k, group;
    unsigned flags;             /* MOE_RENORM or 0 */
    int32_t *topk_idx;          /* device [T][k] */
    float *topk_w;              /* device [T][k] */
    int32_t *counts, *offsets, *perm, *inv_perm;   /* device, as moe_permute */
    void *route_ws;
    size_t route_ws_bytes;
    int regime;                 /* MOE_REGIME_* */
    void *y;
    int y_dtype, y_slices;
    void *ffn_ws;
    size_t ffn_ws_bytes;
    const float *shared_f32;    /* device fp32 [T][H] or NULL */
    const void *residual_f16;   /* device fp16 [T][H] or NULL */
    void *out_f16;              /* device fp16 [T][H] */
    int32_t *host_ids;          /* pinned host int32 [T*k] */
} moe_pool_layer_args;

int moe_pool_layer_forward(moe_pool_t pool, int layer, const moe_pool_layer_args *args,
                           hipStream_t stream, moe_pool_stats_t *step);

/* Cumulative counters since creation or the last reset. */
int moe_pool_stats(moe_pool_t pool, moe_pool_stats_t *out);

/*
 * Per-(layer, expert) access counts since creation or the last reset: the
 * uses of each expert that found it resident and those that copied it in.
 * Their sum over a layer is that layer's routed distinct experts over all
 * its generations.  This is the data a live map of expert traffic is drawn
 * from (Strata, "Tracking MoE expert residency": aggregate hit rates did not
 * explain the behaviour; the per-layer, per-expert distribution did).
 * hits, misses: host int64 arrays of layers*experts, index l*E + e, written.
 * MOE_EINVAL on a null argument.  Host only: nothing waits for the device.
 */
int moe_pool_access_counts(moe_pool_t pool, int64_t *hits, int64_t *misses);

/* Waits for all pool work, restores the initial placement, clears counters. */
int moe_pool_reset(moe_pool_t pool);

/* Waits for all pool work and frees everything.  NULL is a no-op. */
int moe_pool_destroy(moe_pool_t pool);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
