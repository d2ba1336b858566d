/*
 * moe_oracle.c -- plain, slow CPU oracle of the W4A16 MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
 * Python binding) may include, link, load or call this file; only the tests,
 * the smoke check and the benchmark's CPU-baseline leg do.  It shares no code
 * with the HIP path: its fp16 codec, quantiser, blob reader, router, sort,
 * FFN, combine and residency-policy simulator are all written here from the
 * pages and the readings recorded in the design notes.
 *
 * Sources (web pages):
 *  [HR] Horizon RunMap, "Prévia Técnica" (horizonrunmap.com/pt):
 *       "02 / A solução" and "03 / Arquitetura" (router picks experts; the
 *       expert kernel combines compact INT4 weights and FP16 scales with FP16
 *       activations and hands the result back to the model), "08 /
 *       Comportamento do modelo" (W4: INT4 expert weights with FP16 scales;
 *       A16: FP16 activations; FP32 accumulation with explicit roundings),
 *       "03 / Arquitetura, resident-qpacked-cache-v1" (slot cache contract).
 *  [ST] Hamidun News, "Desenvolvedor do Strata cria mapa ao vivo de 24 576
 *       especialistas MoE em uma GTX 1070", section "Como 125 bilhões de
 *       parâmetros cabem em 8 GB" (decayed access counter, LRU/LFU cache).
 *  [LH] lucashiago.com.br local-inference explainer, step 1 formula
 *       (bytes = P x bits / 8, per-block scale overhead).
 *
 * Where the pages are silent (softmax form, tie-break, SwiGLU, group size,
 * quantiser rounding, nibble order, logit summation order, eviction
 * constants) the code follows the readings listed in the design notes; each
 * such point is marked READING below.
 *
 * Precision: everything is fp64 except (a) the router logits, which are
 * defined by a pinned fp32 summation order so that a GPU can reproduce them
 * bit for bit, and (b) the quantiser, whose codes are decided in fp32 like
 * the GPU quantiser.  Only the final layer output is rounded to fp16 (RNE).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fopenmp moe_oracle.c -lm
 * (OpenMP only spreads independent rows over threads; see oracle_set_threads).
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-3)

/* ------------------------------------------------------------------ fp16 */

/* IEEE binary16 -> double, exact. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 31;
    int man = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* subnormal or zero */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);    /* (1 + m/1024) 2^(ex-15) */
    return sign ? -v : v;
}

/* Decode table of all 65536 fp16 values (filled once from the function
 * above; lookups return exactly the same doubles).  Filled before any
 * parallel region starts, so worker threads only read it. */
static double f16tab[65536];
static int f16tab_ready = 0;

static void f16tab_init(void)
{
    if (!f16tab_ready) {
        for (int i = 0; i < 65536; i++)
            f16tab[i] = oracle_f16_to_f64((uint16_t)i);
        f16tab_ready = 1;
    }
}

static double H2D(uint16_t h)
{
    f16tab_init();
    return f16tab[h];
}

/* ------------------------------------------------------------- threads */

/*
 * Worker threads for the per-row loops below (route: tokens; expert FFN:
 * sorted rows; shared FFN: tokens).  Every row is computed by one thread with
 * exactly the same operations in the same order as with one thread, so the
 * results do not depend on the thread count; only the wall time does.
 * n <= 0 restores the OpenMP default.  Without OpenMP everything runs on one
 * thread.
 */
static int or_threads = 0;

void oracle_set_threads(int n) { or_threads = n > 0 ? n : 0; }

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return or_threads > 0 ? or_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* double -> IEEE binary16, round to nearest, ties to even. */
uint16_t oracle_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (a >= 65520.0)                 /* halfway between 65504 and 2^16 -> even = inf */
        return sign | 0x7c00;
    int q_exp;                        /* value = r * 2^q_exp with integer r */
    if (a >= ldexp(1.0, -14)) {
        int e;
        frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
        q_exp = e - 11;               /* 10 fraction bits below the leading one */
    } else {
        q_exp = -24;                  /* subnormal quantum */
    }
    double r = nearbyint(ldexp(a, -q_exp));   /* exact scaling, then RNE */
    if (q_exp == -24)                 /* r in [0, 1024]; 1024 encodes 2^-14 */
        return sign | (uint16_t)r;
    if (r >= 2048.0) {                /* mantissa overflow: next binade */
        r = 1024.0;
        q_exp += 1;
    }
    int ex = q_exp + 25;
    if (ex >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(ex << 10) | (uint16_t)((int)r - 1024);
}

/* ----------------------------------------------------- expert blob format */

/*
 * Canonical expert blob ([HR] "02 / A solução": compact weights and FP16
 * scales kept in separate formats).  Six sections, each starting on a 256-byte
 * boundary:
 *   gate_q [I][H/2], up_q [I][H/2], down_q [H][I/2]        (u8, two codes/byte)
 *   gate_s [I][H/g], up_s [I][H/g], down_s [H][I/g]        (fp16 scales)
 * Rows are [out][in] with the input dimension contiguous.  Byte b of a row
 * holds element 2b in its low nibble and element 2b+1 in its high nibble, as
 * u = q + 8 (READING: symmetric codes q in [-7, 7], no zero point).
 */
static int64_t al256(int64_t x) { return (x + 255) & ~(int64_t)255; }

int oracle_blob_layout(int H, int I, int g, int64_t off[6], int64_t *total)
{
    if (H <= 0 || I <= 0 || g <= 0 || H % g || I % g || H % 2 || I % 2)
        return OR_EINVAL;
    int64_t sz[6];
    sz[0] = (int64_t)I * H / 2;
    sz[1] = (int64_t)I * H / 2;
    sz[2] = (int64_t)H * I / 2;
    sz[3] = (int64_t)I * (H / g) * 2;
    sz[4] = (int64_t)I * (H / g) * 2;
    sz[5] = (int64_t)H * (I / g) * 2;
    int64_t o = 0;
    for (int i = 0; i < 6; i++) {
        off[i] = o;
        o = al256(o + sz[i]);
    }
    *total = o;
    return OR_OK;
}

/* ------------------------------------------------------------- quantiser */

/*
 * Group-wise symmetric INT4 quantisation of a [rows][K] fp32 matrix, groups of
 * g consecutive elements along K ([HR] "08": expert weights INT4 with FP16
 * scales; [LH] step 1: every block carries its own scale).
 * READING: s = fp16_rne(amax / 7) with amax/7 computed in fp32;
 *          q = clamp(rne(w / s), -7, 7) with w / s computed in fp32;
 *          q = 0 when s == 0.
 * Codes are decided in fp32 so a GPU quantiser can make the same decision.
 */
int oracle_quantize_rows(const float *w, int rows, int K, int g,
                         uint8_t *q, uint16_t *s)
{
    if (!w || !q || !s || rows < 0 || K <= 0 || g <= 0 || K % g || K % 2)
        return OR_EINVAL;
    int ng = K / g;
    for (int r = 0; r < rows; r++) {
        const float *wr = w + (int64_t)r * K;
        uint8_t *qr = q + (int64_t)r * (K / 2);
        memset(qr, 0, (size_t)(K / 2));
        for (int G = 0; G < ng; G++) {
            float amax = 0.0f;
            for (int i = 0; i < g; i++) {
                float a = fabsf(wr[G * g + i]);
                if (a > amax)
                    amax = a;
            }
            float sf = amax / 7.0f;
            uint16_t sh = oracle_f64_to_f16((double)sf);
            s[(int64_t)r * ng + G] = sh;
            float sv = (float)oracle_f16_to_f64(sh);
            for (int i = 0; i < g; i++) {
                int c = G * g + i;
                int qi = 0;
                if (sv != 0.0f) {
                    float t = wr[c] / sv;
                    double rr = nearbyint((double)t);
                    if (rr > 7.0) rr = 7.0;
                    if (rr < -7.0) rr = -7.0;
                    qi = (int)rr;
                }
                uint8_t u = (uint8_t)(qi + 8);
                if (c & 1)
                    qr[c / 2] |= (uint8_t)(u << 4);
                else
                    qr[c / 2] |= u;
            }
        }
    }
    return OR_OK;
}

/* Quantise one expert's three projections into a canonical blob. */
int oracle_pack_expert(const float *wg, const float *wu, const float *wd,
                       int H, int I, int g, uint8_t *blob)
{
    int64_t off[6], total;
    int rc = oracle_blob_layout(H, I, g, off, &total);
    if (rc) return rc;
    memset(blob, 0, (size_t)total);
    rc = oracle_quantize_rows(wg, I, H, g, blob + off[0], (uint16_t *)(blob + off[3]));
    if (rc) return rc;
    rc = oracle_quantize_rows(wu, I, H, g, blob + off[1], (uint16_t *)(blob + off[4]));
    if (rc) return rc;
    return oracle_quantize_rows(wd, H, I, g, blob + off[2], (uint16_t *)(blob + off[5]));
}

/* Dequantised element (r, c) of a [rows][K] section: q * s, exact in fp64. */
static double deq(const uint8_t *qs, const uint16_t *ss, int K, int g, int r, int c)
{
    uint8_t b = qs[(int64_t)r * (K / 2) + c / 2];
    int u = (c & 1) ? (b >> 4) : (b & 15);
    return (double)(u - 8) * H2D(ss[(int64_t)r * (K / g) + c / g]);
}

/* Dequantise a whole [rows][K] section to fp64 (tests use it as a pin). */
int oracle_dequant_rows(const uint8_t *q, const uint16_t *s, int rows, int K, int g,
                        double *out)
{
    if (!q || !s || !out || K % g || K % 2)
        return OR_EINVAL;
    for (int r = 0; r < rows; r++)
        for (int c = 0; c < K; c++)
            out[(int64_t)r * K + c] = deq(q, s, K, g, r, c);
    return OR_OK;
}

/* ------------------------------------------- zero-point (asymmetric) INT4 */

/*
 * Asymmetric variant of the format: the local-inference explainer's step 1
 * ([LH], the file-size formula) gives every block of weights a scale and a
 * zero point.  Canonical blob: the six sections above (codes and fp16
 * scales, same places) followed by three more, each 256-byte aligned:
 *   gate_z [I][H/g], up_z [I][H/g], down_z [H][I/g]    (u8, one per group)
 * A stored nibble u in [0, 15] means W = (u - z) * s.  (The symmetric format
 * is the case z = 8 for every group.)
 */
int oracle_blob_layout_zp(int H, int I, int g, int64_t off[9], int64_t *total)
{
    int64_t o6[6], t6;
    int rc = oracle_blob_layout(H, I, g, o6, &t6);
    if (rc)
        return rc;
    for (int i = 0; i < 6; i++)
        off[i] = o6[i];
    int64_t sz[3] = {(int64_t)I * (H / g), (int64_t)I * (H / g), (int64_t)H * (I / g)};
    int64_t o = t6;
    for (int i = 0; i < 3; i++) {
        off[6 + i] = o;
        o = al256(o + sz[i]);
    }
    *total = o;
    return OR_OK;
}

/*
 * Group-wise asymmetric INT4 quantisation of a [rows][K] fp32 matrix.
 * READING (the explainer names the zero point, not its rule; this is the
 * usual min/max affine rule, with zero kept inside the range):
 *   lo = min(min w, 0), hi = max(max w, 0)                   (fp32)
 *   s  = fp16_rne((hi - lo) / 15), the quotient in fp32
 *   z  = clamp(rne(-lo / s), 0, 15), the quotient in fp32
 *   u  = clamp(rne(w / s) + z, 0, 15), w / s in fp32
 *   s == 0 (an all-zero group): z = 0 and u = 0.
 * Codes are decided in fp32 so a GPU quantiser can make the same decisions.
 */
int oracle_quantize_rows_zp(const float *w, int rows, int K, int g,
                            uint8_t *q, uint16_t *s, uint8_t *z)
{
    if (!w || !q || !s || !z || rows < 0 || K <= 0 || g <= 0 || K % g || K % 2)
        return OR_EINVAL;
    int ng = K / g;
    for (int r = 0; r < rows; r++) {
        const float *wr = w + (int64_t)r * K;
        uint8_t *qr = q + (int64_t)r * (K / 2);
        memset(qr, 0, (size_t)(K / 2));
        for (int G = 0; G < ng; G++) {
            float lo = 0.0f, hi = 0.0f;
            for (int i = 0; i < g; i++) {
                float v = wr[G * g + i];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            float sf = (hi - lo) / 15.0f;
            uint16_t sh = oracle_f64_to_f16((double)sf);
            s[(int64_t)r * ng + G] = sh;
            float sv = (float)oracle_f16_to_f64(sh);
            int zi = 0;
            if (sv != 0.0f) {
                float t = -lo / sv;
                double rz = nearbyint((double)t);
                if (rz < 0.0) rz = 0.0;
                if (rz > 15.0) rz = 15.0;
                zi = (int)rz;
            }
            z[(int64_t)r * ng + G] = (uint8_t)zi;
            for (int i = 0; i < g; i++) {
                int c = G * g + i;
                int ui = 0;
                if (sv != 0.0f) {
                    float t = wr[c] / sv;
                    double ru = nearbyint((double)t) + zi;
                    if (ru < 0.0) ru = 0.0;
                    if (ru > 15.0) ru = 15.0;
                    ui = (int)ru;
                }
                if (c & 1)
                    qr[c / 2] |= (uint8_t)(ui << 4);
                else
                    qr[c / 2] |= (uint8_t)ui;
            }
        }
    }
    return OR_OK;
}

/* Quantise one expert's three projections into a zero-point canonical blob. */
int oracle_pack_expert_zp(const float *wg, const float *wu, const float *wd,
                          int H, int I, int g, uint8_t *blob)
{
    int64_t off[9], total;
    int rc = oracle_blob_layout_zp(H, I, g, off, &total);
    if (rc) return rc;
    memset(blob, 0, (size_t)total);
    rc = oracle_quantize_rows_zp(wg, I, H, g, blob + off[0], (uint16_t *)(blob + off[3]),
                                 blob + off[6]);
    if (rc) return rc;
    rc = oracle_quantize_rows_zp(wu, I, H, g, blob + off[1], (uint16_t *)(blob + off[4]),
                                 blob + off[7]);
    if (rc) return rc;
    return oracle_quantize_rows_zp(wd, H, I, g, blob + off[2], (uint16_t *)(blob + off[5]),
                                   blob + off[8]);
}

/* Dequantised element (r, c) of a zero-point [rows][K] section: (u - z) * s,
 * exact in fp64. */
static double deq_zp(const uint8_t *qs, const uint16_t *ss, const uint8_t *zs, int K, int g,
                     int r, int c)
{
    uint8_t b = qs[(int64_t)r * (K / 2) + c / 2];
    int u = (c & 1) ? (b >> 4) : (b & 15);
    int64_t G = (int64_t)r * (K / g) + c / g;
    return (double)(u - (int)zs[G]) * H2D(ss[G]);
}

int oracle_dequant_rows_zp(const uint8_t *q, const uint16_t *s, const uint8_t *z, int rows,
                           int K, int g, double *out)
{
    if (!q || !s || !z || !out || K % g || K % 2)
        return OR_EINVAL;
    for (int r = 0; r < rows; r++)
        for (int c = 0; c < K; c++)
            out[(int64_t)r * K + c] = deq_zp(q, s, z, K, g, r, c);
    return OR_OK;
}

/* ---------------------------------------------------------------- router */

/*
 * Router logit l[t,e] = sum_h x[t,h] * Wr[e,h] in fp32, in a pinned order
 * (READING; the pages only say accumulation is FP32 with explicit roundings,
 * [HR] "08"): H is cut into chunks of 8 elements; chunk c is added, element
 * by element in increasing h, into partial number (c mod 64), chunks taken in
 * increasing c; the 64 partials are then combined by an xor butterfly with
 * strides 32, 16, 8, 4, 2, 1 (a_j <- a_j + a_{j xor s}).  fp16 x fp16
 * products are exact in fp32, so this order fixes every rounding.
 */
static float logit_pinned(const float *x, const float *w, int H)
{
    float part[64], nxt[64];
    for (int j = 0; j < 64; j++)
        part[j] = 0.0f;
    for (int c = 0; c < H / 8; c++) {
        int lane = c % 64;
        for (int i = 0; i < 8; i++) {
            int h = c * 8 + i;
            float prod = x[h] * w[h];
            part[lane] = part[lane] + prod;
        }
    }
    for (int st = 32; st >= 1; st >>= 1) {
        for (int j = 0; j < 64; j++)
            nxt[j] = part[j] + part[j ^ st];
        memcpy(part, nxt, sizeof part);
    }
    return part[0];
}

/*
 * Routing ([HR] "03 / Arquitetura": the router chooses which experts work on
 * this token).  READING: logits over all E experts (plus an optional fp32
 * per-expert bias added after the dot product); the top-k are the k largest
 * logits, ties going to the lower expert index, stored in that order;
 * weights are softmax over all E logits (fp64) taken at the chosen experts,
 * not renormalised unless `renorm` is set.
 * Outputs: idx[T][k] int32, w[T][k] fp32, optionally logits[T][E] fp32.
 */
/* Top-k, softmax weights and optional logits of one token (the steps of
 * oracle_route below; l, p, taken are scratch of E entries). */
static void route_token(const float *xf, const float *wf, const float *bias, int H, int E,
                        int k, int renorm, float *l, double *p, char *taken, int32_t *idx,
                        float *w, float *logits)
{
    for (int e = 0; e < E; e++) {
        float v = logit_pinned(xf, wf + (int64_t)e * H, H);
        if (bias)
            v = v + bias[e];
        l[e] = v;
        if (logits)
            logits[e] = v;
    }
    /* top-k by (logit descending, index ascending) */
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++) {
            if (taken[e])
                continue;
            if (best < 0 || l[e] > l[best])
                best = e;
        }
        taken[best] = 1;
        idx[j] = best;
    }
    /* softmax over all E, fp64 */
    double m = l[0];
    for (int e = 1; e < E; e++)
        if (l[e] > m) m = l[e];
    double den = 0.0;
    for (int e = 0; e < E; e++) {
        p[e] = exp((double)l[e] - m);
        den += p[e];
    }
    double sel = 0.0;
    for (int j = 0; j < k; j++)
        sel += p[idx[j]] / den;
    for (int j = 0; j < k; j++) {
        double pj = p[idx[j]] / den;
        if (renorm)
            pj = pj / sel;
        w[j] = (float)pj;
    }
}

int oracle_route(const uint16_t *x, const uint16_t *wr, const float *bias,
                 int T, int H, int E, int k, int renorm,
                 int32_t *idx, float *w, float *logits)
{
    if (!x || !wr || !idx || !w || T < 0 || H <= 0 || H % 8 || E <= 0 || k <= 0 || k > E)
        return OR_EINVAL;
    f16tab_init();
    float *wf = malloc(sizeof(float) * (size_t)E * H);   /* fp16 values, exact in fp32 */
    if (!wf)
        return OR_ENOMEM;
    for (int64_t i = 0; i < (int64_t)E * H; i++)
        wf[i] = (float)H2D(wr[i]);
    int rc = OR_OK;
#pragma omp parallel num_threads(oracle_get_threads()) if (T > 1)
    {
        float *l = malloc(sizeof(float) * (size_t)E);
        double *p = malloc(sizeof(double) * (size_t)E);
        char *taken = malloc((size_t)E);
        float *xf = malloc(sizeof(float) * (size_t)H);
        int ok = l && p && taken && xf;
        if (!ok) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        }
#pragma omp for schedule(static)
        for (int t = 0; t < T; t++) {
            if (!ok)
                continue;
            for (int h = 0; h < H; h++)
                xf[h] = (float)H2D(x[(int64_t)t * H + h]);
            route_token(xf, wf, bias, H, E, k, renorm, l, p, taken, idx + (int64_t)t * k,
                        w + (int64_t)t * k, logits ? logits + (int64_t)t * E : NULL);
        }
        free(l); free(p); free(taken); free(xf);
    }
    free(wf);
    return rc;
}

/* ----------------------------------------------------------- permutation */

/*
 * Token-to-expert grouping (the pages' "experts computed in groups", [HR]
 * "04 / Resultados", Grouped executor).  READING: stable counting sort of
 * the flat index f = t*k + j by expert idx[f]:
 *   counts[e], offsets[E+1] (exclusive scan, offsets[E] = T*k),
 *   perm[p] = f for sorted position p (f ascending inside each expert),
 *   inv_perm[f] = p.
 */
int oracle_permute(const int32_t *idx, int T, int k, int E,
                   int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm)
{
    if (!idx || !counts || !offsets || !perm || !inv_perm || T < 0 || k <= 0 || E <= 0)
        return OR_EINVAL;
    int n = T * k;
    for (int e = 0; e < E; e++)
        counts[e] = 0;
    for (int f = 0; f < n; f++) {
        if (idx[f] < 0 || idx[f] >= E)
            return OR_EINVAL;
        counts[idx[f]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = malloc(sizeof(int32_t) * (size_t)E);
    if (!fill)
        return OR_ENOMEM;
    for (int e = 0; e < E; e++)
        fill[e] = offsets[e];
    for (int f = 0; f < n; f++) {
        int p = fill[idx[f]]++;
        perm[p] = f;
        inv_perm[f] = p;
    }
    free(fill);
    return OR_OK;
}

/* ------------------------------------------------------------ expert FFN */

static double silu(double a) { return a / (1.0 + exp(-a)); }

/*
 * Routed expert FFN straight from the compact weights ([HR] "03": the kernel
 * reads compact weights and scales, uses the FP16 activations and never keeps
 * an expanded expert; here each element is decoded on use).  READING: SwiGLU,
 *   h = silu(Wg x) * (Wu x),  y = Wd h,  W = q * s,  all in fp64.
 * W is decoded per the blob format fmt: 0 symmetric ((u - 8) s), 1 zero
 * point ((u - z) s, oracle_blob_layout_zp).
 * Sorted row p (offsets[e] <= p < offsets[e+1]) belongs to expert e and to
 * token t = perm[p] / k.  `rows` (length nrows) selects sorted rows to
 * compute; NULL means all T*k rows.  y is [nrows][H] fp64.
 */
int oracle_expert_ffn_fmt(const uint16_t *x, const int32_t *perm, const int32_t *offsets,
                          const uint8_t *const *blobs, int T, int H, int I, int E, int k, int g,
                          int fmt, const int32_t *rows, int nrows, double *y)
{
    int64_t off[9], total;
    if (!x || !perm || !offsets || !blobs || !y || k <= 0 || (fmt != 0 && fmt != 1))
        return OR_EINVAL;
    if (fmt == 1 ? oracle_blob_layout_zp(H, I, g, off, &total)
                 : oracle_blob_layout(H, I, g, off, &total))
        return OR_EINVAL;
    f16tab_init();
    int n = T * k;
    if (!rows)
        nrows = n;
    /* expert of every requested row, checked before any arithmetic */
    int *ex = malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    if (!ex)
        return OR_ENOMEM;
    for (int r = 0; r < nrows; r++) {
        int p = rows ? rows[r] : r;
        int e = 0;
        if (p >= 0 && p < n)
            while (e < E && !(offsets[e] <= p && p < offsets[e + 1]))
                e++;
        if (p < 0 || p >= n || e == E || !blobs[e]) {
            free(ex);
            return OR_EINVAL;
        }
        ex[r] = e;
    }
    int rc = OR_OK;
    /* rows in contiguous runs per thread: sorted rows of one expert stay
     * together, so each thread decodes few experts */
#pragma omp parallel num_threads(oracle_get_threads()) if (nrows > 1)
    {
        double *xv = malloc(sizeof(double) * (size_t)H);
        double *hv = malloc(sizeof(double) * (size_t)I);
        /* dequantised matrices of the expert in use (decoded once per expert) */
        double *Wg = malloc(sizeof(double) * (size_t)I * H);
        double *Wu = malloc(sizeof(double) * (size_t)I * H);
        double *Wd = malloc(sizeof(double) * (size_t)H * I);
        int ok = xv && hv && Wg && Wu && Wd, cur = -1;
        if (!ok) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        }
#pragma omp for schedule(static)
        for (int r = 0; r < nrows; r++) {
            if (!ok)
                continue;
            int p = rows ? rows[r] : r;
            int e = ex[r];
            if (e != cur) {
                const uint8_t *b = blobs[e];
                const uint8_t *gq = b + off[0], *uq = b + off[1], *dq = b + off[2];
                const uint16_t *gs = (const uint16_t *)(b + off[3]);
                const uint16_t *us = (const uint16_t *)(b + off[4]);
                const uint16_t *ds = (const uint16_t *)(b + off[5]);
                const uint8_t *gz = fmt ? b + off[6] : NULL, *uz = fmt ? b + off[7] : NULL,
                              *dz = fmt ? b + off[8] : NULL;
                for (int i = 0; i < I; i++)
                    for (int c = 0; c < H; c++) {
                        Wg[(int64_t)i * H + c] = fmt ? deq_zp(gq, gs, gz, H, g, i, c)
                                                     : deq(gq, gs, H, g, i, c);
                        Wu[(int64_t)i * H + c] = fmt ? deq_zp(uq, us, uz, H, g, i, c)
                                                     : deq(uq, us, H, g, i, c);
                    }
                for (int o = 0; o < H; o++)
                    for (int i = 0; i < I; i++)
                        Wd[(int64_t)o * I + i] = fmt ? deq_zp(dq, ds, dz, I, g, o, i)
                                                     : deq(dq, ds, I, g, o, i);
                cur = e;
            }
            int t = perm[p] / k;
            for (int c = 0; c < H; c++)
                xv[c] = H2D(x[(int64_t)t * H + c]);
            for (int i = 0; i < I; i++) {
                double a = 0.0, u = 0.0;
                const double *wg = Wg + (int64_t)i * H, *wu = Wu + (int64_t)i * H;
                for (int c = 0; c < H; c++) {
                    a += wg[c] * xv[c];
                    u += wu[c] * xv[c];
                }
                hv[i] = silu(a) * u;
            }
            for (int o = 0; o < H; o++) {
                double acc = 0.0;
                const double *wd = Wd + (int64_t)o * I;
                for (int i = 0; i < I; i++)
                    acc += wd[i] * hv[i];
                y[(int64_t)r * H + o] = acc;
            }
        }
        free(xv); free(hv); free(Wg); free(Wu); free(Wd);
    }
    free(ex);
    return rc;
}

/* The symmetric format (z = 8): the entry point the tests use by default. */
int oracle_expert_ffn(const uint16_t *x, const int32_t *perm, const int32_t *offsets,
                      const uint8_t *const *blobs, int T, int H, int I, int E, int k, int g,
                      const int32_t *rows, int nrows, double *y)
{
    return oracle_expert_ffn_fmt(x, perm, offsets, blobs, T, H, I, E, k, g, 0, rows, nrows, y);
}

/*
 * Shared (non-routed) expert in FP16 weights ([HR] "03": the non-routed part
 * stays outside the INT4 compression, in FP16).  READING: the same SwiGLU FFN,
 * weights wg, wu [Is][H] and wd [H][Is] fp16 row-major, evaluated in fp64 for
 * the tokens in `toks` (NULL = all T).  s is [ntoks][H] fp64.
 */
int oracle_shared_ffn(const uint16_t *x, const uint16_t *wg, const uint16_t *wu,
                      const uint16_t *wd, int T, int H, int Is,
                      const int32_t *toks, int ntoks, double *s)
{
    if (!x || !wg || !wu || !wd || !s || H <= 0 || Is <= 0)
        return OR_EINVAL;
    f16tab_init();
    if (!toks)
        ntoks = T;
    int rc = OR_OK;
#pragma omp parallel num_threads(oracle_get_threads()) if (ntoks > 1)
    {
        double *xv = malloc(sizeof(double) * (size_t)H);
        double *hv = malloc(sizeof(double) * (size_t)Is);
        int ok = xv && hv;
        if (!ok) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        }
#pragma omp for schedule(static)
        for (int r = 0; r < ntoks; r++) {
            if (!ok)
                continue;
            int t = toks ? toks[r] : r;
            for (int c = 0; c < H; c++)
                xv[c] = H2D(x[(int64_t)t * H + c]);
            for (int i = 0; i < Is; i++) {
                double a = 0.0, u = 0.0;
                for (int c = 0; c < H; c++) {
                    a += H2D(wg[(int64_t)i * H + c]) * xv[c];
                    u += H2D(wu[(int64_t)i * H + c]) * xv[c];
                }
                hv[i] = silu(a) * u;
            }
            for (int o = 0; o < H; o++) {
                double acc = 0.0;
                for (int i = 0; i < Is; i++)
                    acc += H2D(wd[(int64_t)o * Is + i]) * hv[i];
                s[(int64_t)r * H + o] = acc;
            }
        }
        free(xv); free(hv);
    }
    return rc;
}

/*
 * Shared-expert gate.  The pages name a second model whose layers have 60
 * routed experts with a top-4 executor ([HR] "Prévia Técnica", the
 * top4-fused-v1 rows of the residency results) but print no layer shape and no
 * form of its shared path.  READING: that model family scales its shared
 * expert's output, per token, by a sigmoid of one more linear function of the
 * token, g_t = 1 / (1 + exp(-sum_c x[t,c] * wsg[c])), wsg an fp16 vector of
 * length H with no bias.  Evaluated in fp64 for the tokens in `toks` (NULL =
 * all T); gate is [ntoks].
 */
int oracle_shared_gate(const uint16_t *x, const uint16_t *wsg, int T, int H,
                       const int32_t *toks, int ntoks, double *gate)
{
    if (!x || !wsg || !gate || H <= 0 || T < 0)
        return OR_EINVAL;
    if (!toks)
        ntoks = T;
    for (int r = 0; r < ntoks; r++) {
        int t = toks ? toks[r] : r;
        double a = 0.0;
        for (int c = 0; c < H; c++)
            a += H2D(x[(int64_t)t * H + c]) * H2D(wsg[c]);
        gate[r] = 1.0 / (1.0 + exp(-a));
    }
    return OR_OK;
}

/* --------------------------------------------------------------- combine */

/*
 * Router-weighted combine ([HR] "03": the expert results go back to the rest
 * of the model weighted by the router).  READING:
 *   out[t] = fp16_rne( residual[t] + sum_j w[t,j] * y[inv_perm[t*k+j]] + G_t s[t] )
 * evaluated in fp64; residual (fp16) and s (fp64) are optional (NULL).  G_t
 * is shared_gate[t] when a gate is given (the gated shared expert above),
 * else 1.  y is indexed by sorted row: [T*k][H].  out_f64 (optional) gets the
 * value before the final rounding.
 */
int oracle_combine(const double *y, const int32_t *inv_perm, const float *w,
                   const double *shared, const double *shared_gate,
                   const uint16_t *residual, int T, int H, int k, uint16_t *out,
                   double *out_f64)
{
    if (!y || !inv_perm || !w || !out || T < 0 || H <= 0 || k <= 0)
        return OR_EINVAL;
    for (int t = 0; t < T; t++) {
        for (int o = 0; o < H; o++) {
            double acc = residual ? H2D(residual[(int64_t)t * H + o]) : 0.0;
            for (int j = 0; j < k; j++) {
                int p = inv_perm[(int64_t)t * k + j];
                acc += (double)w[(int64_t)t * k + j] * y[(int64_t)p * H + o];
            }
            if (shared)
                acc += (shared_gate ? shared_gate[t] : 1.0) * shared[(int64_t)t * H + o];
            out[(int64_t)t * H + o] = oracle_f64_to_f16(acc);
            if (out_f64)
                out_f64[(int64_t)t * H + o] = acc;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------- residency simulator */

/*
 * Replays a routing trace through the expert-slot cache policy.
 * [HR] "03 / Arquitetura" (resident-qpacked-cache-v1): capacity is fixed
 * before requests; misses are copied into spare slots while readers keep the
 * previous generation; evicted copies are dropped (never written back).
 * [ST] "Como 125 bilhões...": eviction by an access counter whose old hits
 * decay (an LRU/LFU hybrid).
 * READING of the policy, per routed event (layer l, k distinct experts R):
 *   1. decay every counter of layer l: c <- c - (c >> shift)
 *      (shift < 0: no decay, i.e. LFU);
 *   2. c[e] += 65536 for e in R;
 *   3. hits (R resident) are touched in ascending expert id, each taking the
 *      next value of a global use clock;
 *   4. misses are handled in ascending expert id: the victim is the resident
 *      expert not in R with the lowest (counter, last use, id); the miss takes
 *      its place and the next clock value.
 * Initial placement per layer is experts 0..C-1 with last-use values ordered
 * by id (expert 0 oldest).  shift = 0 is plain LRU.
 * Outputs per event: hits, misses, the missed experts and the victims in the
 * order handled (-1 padded to k).
 */
int oracle_pool_sim(int L, int E, int C, int shift, int k,
                    const int32_t *ev_layer, const int32_t *ev_ids, int n_ev,
                    int32_t *ev_hits, int32_t *ev_misses,
                    int32_t *miss_list, int32_t *evict_list)
{
    if (L <= 0 || E <= 0 || C < k || C > E || k <= 0 || !ev_layer || !ev_ids)
        return OR_EINVAL;
    size_t n = (size_t)L * E;
    char *res = calloc(n, 1);
    int64_t *cnt = calloc(n, sizeof(int64_t));
    int64_t *last = calloc(n, sizeof(int64_t));
    char *inR = calloc((size_t)E, 1);
    if (!res || !cnt || !last || !inR) {
        free(res); free(cnt); free(last); free(inR);
        return OR_ENOMEM;
    }
    for (int l = 0; l < L; l++)
        for (int e = 0; e < C; e++) {
            res[(size_t)l * E + e] = 1;
            last[(size_t)l * E + e] = (int64_t)e - C;
        }
    int64_t clock = 0;
    int rc = OR_OK;
    for (int i = 0; i < n_ev; i++) {
        int l = ev_layer[i];
        const int32_t *R = ev_ids + (int64_t)i * k;
        if (l < 0 || l >= L) { rc = OR_EINVAL; break; }
        char *rl = res + (size_t)l * E;
        int64_t *cl = cnt + (size_t)l * E, *tl = last + (size_t)l * E;
        memset(inR, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            if (R[j] < 0 || R[j] >= E || inR[R[j]]) { rc = OR_EINVAL; break; }
            inR[R[j]] = 1;
        }
        if (rc) break;
        if (shift >= 0)
            for (int e = 0; e < E; e++)
                cl[e] -= cl[e] >> shift;
        for (int e = 0; e < E; e++)
            if (inR[e])
                cl[e] += 65536;
        int hits = 0, misses = 0;
        for (int e = 0; e < E; e++)
            if (inR[e] && rl[e]) {
                tl[e] = ++clock;
                hits++;
            }
        for (int e = 0; e < E; e++) {
            if (!inR[e] || rl[e])
                continue;
            int v = -1;
            for (int c = 0; c < E; c++) {
                if (!rl[c] || inR[c])
                    continue;
                if (v < 0 || cl[c] < cl[v] || (cl[c] == cl[v] && tl[c] < tl[v]) ||
                    (cl[c] == cl[v] && tl[c] == tl[v] && c < v))
                    v = c;
            }
            rl[v] = 0;
            rl[e] = 1;
            tl[e] = ++clock;
            if (miss_list) miss_list[(int64_t)i * k + misses] = e;
            if (evict_list) evict_list[(int64_t)i * k + misses] = v;
            misses++;
        }
        for (int j = misses; j < k; j++) {
            if (miss_list) miss_list[(int64_t)i * k + j] = -1;
            if (evict_list) evict_list[(int64_t)i * k + j] = -1;
        }
        if (ev_hits) ev_hits[i] = hits;
        if (ev_misses) ev_misses[i] = misses;
    }
    free(res); free(cnt); free(last); free(inR);
    return rc;
}

/*
 * Profile-pinned residency ([LH] step 4: with VRAM for only part of the
 * experts there are two obvious policies, keeping what was used last or
 * measuring usage beforehand and fixing the most used; the profile needs a
 * measurement pass and ages when the subject changes; no policy beats the
 * summed probability of the experts that fit without guessing the future).
 * READING: the profile is the number of routed events per (layer, expert) in a
 * measurement pass; layer l pins the C experts with the highest counts (ties
 * to the lower id), listed in ascending id in pinned[l*C .. l*C+C).
 */
int oracle_profile_pin(const int64_t *counts, int L, int E, int C, int32_t *pinned)
{
    if (!counts || !pinned || L <= 0 || E <= 0 || C <= 0 || C > E)
        return OR_EINVAL;
    char *take = malloc((size_t)E);
    if (!take)
        return OR_ENOMEM;
    for (int l = 0; l < L; l++) {
        const int64_t *c = counts + (size_t)l * E;
        memset(take, 0, (size_t)E);
        for (int i = 0; i < C; i++) {          /* C rounds of "best not yet taken" */
            int b = -1;
            for (int e = 0; e < E; e++)
                if (!take[e] && (b < 0 || c[e] > c[b]))
                    b = e;                       /* strict >: ties keep the lower id */
            take[b] = 1;
        }
        int j = 0;
        for (int e = 0; e < E; e++)
            if (take[e])
                pinned[(size_t)l * C + j++] = e;
    }
    free(take);
    return OR_OK;
}

/*
 * Replays a routing trace through the pinned policy.  READING: a routed
 * expert in the layer's pinned set is a hit; every other routed expert is a
 * miss, copied for that event only (the next use pays again); nothing is
 * evicted.  miss_list[i*k ..] gets the misses in ascending id, padded by -1.
 */
int oracle_pool_sim_pinned(int L, int E, int C, const int32_t *pinned, int k,
                           const int32_t *ev_layer, const int32_t *ev_ids, int n_ev,
                           int32_t *ev_hits, int32_t *ev_misses, int32_t *miss_list)
{
    if (L <= 0 || E <= 0 || C <= 0 || C > E || k <= 0 || !pinned || !ev_layer || !ev_ids)
        return OR_EINVAL;
    char *res = calloc((size_t)L * E, 1);
    char *inR = calloc((size_t)E, 1);
    if (!res || !inR) {
        free(res); free(inR);
        return OR_ENOMEM;
    }
    int rc = OR_OK;
    for (int l = 0; l < L && !rc; l++)
        for (int i = 0; i < C; i++) {
            int e = pinned[(size_t)l * C + i];
            if (e < 0 || e >= E || res[(size_t)l * E + e]) { rc = OR_EINVAL; break; }
            res[(size_t)l * E + e] = 1;
        }
    for (int i = 0; i < n_ev && !rc; i++) {
        int l = ev_layer[i];
        const int32_t *R = ev_ids + (int64_t)i * k;
        if (l < 0 || l >= L) { rc = OR_EINVAL; break; }
        memset(inR, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            if (R[j] < 0 || R[j] >= E || inR[R[j]]) { rc = OR_EINVAL; break; }
            inR[R[j]] = 1;
        }
        if (rc) break;
        int hits = 0, misses = 0;
        for (int e = 0; e < E; e++) {
            if (!inR[e])
                continue;
            if (res[(size_t)l * E + e])
                hits++;
            else {
                if (miss_list) miss_list[(int64_t)i * k + misses] = e;
                misses++;
            }
        }
        for (int j = misses; j < k; j++)
            if (miss_list) miss_list[(int64_t)i * k + j] = -1;
        if (ev_hits) ev_hits[i] = hits;
        if (ev_misses) ev_misses[i] = misses;
    }
    free(res); free(inR);
    return rc;
}

/* ------------------------------------------------ array helpers (tests) */

void oracle_f16_to_f64_n(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f16_to_f64(in[i]);
}

void oracle_f64_to_f16_n(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f64_to_f16(in[i]);
}
