/*
 * moe_oracle.c -- plain, slow, CPU reference of a mixture-of-experts FFN layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or call this
 * file; only the test-suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes follows the description of the single-GPU ("TP=1, local") MoE kernels in
 * "CuTeDSL at Perplexity" (Perplexity blog), section "Mixture-of-Experts Dispatch/Combine",
 * subsection "Local": a router picks experts per token, dispatch counts the tokens of every
 * expert and gives each token a unique index inside its expert's list, the MoE GEMMs run per
 * expert, and combine accumulates the expert outputs of every token with its routing weight.
 * The pages give no formulas; each step states the reading it takes:
 *
 *  route    logits l[t,e] = sum_h x[t,h] * Wr[e,h] (+ b[e]) in the CANONICAL fp32 order below
 *           (the order is part of the routing contract, so that expert indices are bit-exact);
 *           top-k by (logit descending, expert index ascending); weights = softmax over the k
 *           selected logits (== the full softmax renormalised over the selection), in fp64.
 *  permute  counts[e], exclusive offsets[e], and the STABLE counting sort of assignments
 *           a = t*k + j by expert: sorted_token[pos] = t, inv_perm[a] = pos.
 *  expert   SwiGLU FFN (SiLU(gate) * up, then down), gate rows first in W13; no biases.
 *  combine  y[t] = sum_j w[t,j] * y_perm[inv_perm[t*k+j]].
 *  MXFP8    (OCP microscaling formats v1.0, the MXFP8 scheme "Hosting Qwen on Blackwell" deploys,
 *           section Quantization, and whose 32-element absolute-maximum reductions "CuTeDSL at
 *           Perplexity" mentions, section Blackwell): weights are E4M3 values with one E8M0
 *           scale (2^(s-127)) per 32 consecutive elements along K.  The layer quantizes its
 *           activations the same way on the fly: x before the gate/up projection and hid before
 *           the down projection, each block of 32 along K taking the shared exponent
 *           X = floor(log2(max|v|)) - 8 (8 = the largest E4M3 exponent; X = -127 for an all-zero
 *           block, X clamped to [-127, 127]) and elements v / 2^X clamped to +-448 and rounded to
 *           the nearest E4M3 value, ties to the even code.  What gets quantized are the layer's
 *           bf16 activations: x is bf16 already, and hid, an activation of the layer like x, is
 *           rounded to bf16 (nearest even) first.  Products of decoded values are then
 *           accumulated in double like every other format.
 *  MXFP4    the same layer with E2M1 weights (two per byte, even element in the low nibble):
 *           w = e2m1 * 2^(s-127) with one E8M0 scale s per 32 elements along K; activations
 *           in MXFP8 exactly as above (the pages evaluate MXFP4 weights beside MXFP8).
 *  held     expert parallelism with replicated inputs (same article, same section: with
 *           tensor parallelism the local dispatch selects only the tokens routed to the
 *           experts of the current rank, and the local combine is followed by an all-reduce):
 *           given a held range [eb, ee), permute keeps only assignments whose expert lies in
 *           it (the others get inv_perm = -1 and no row), and combine skips them, so y is the
 *           rank's partial sum.  eb = 0, ee = E is the single-GPU layer.
 *
 * Floating point: every value is decoded exactly into double (its own bf16 / E2M1 / E4M3
 * decoders) and every sum after routing is accumulated in double.  Parity pins: see the tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_NVFP4 = 2, ORC_MXFP8 = 3, ORC_MXFP4 = 4 };

/* ------------------------------------------------------------------------------------ */
/* decoders                                                                              */
/* ------------------------------------------------------------------------------------ */

/* bfloat16: the upper half of an IEEE binary32. */
static float dec_bf16_f(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* E2M1 (OCP microscaling formats v1.0, FP4): sign bit 3, exponent bits 2..1 (bias 1),
 * mantissa bit 0; exponent 0 is subnormal with value mantissa * 2^-1. */
static double dec_e2m1(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP 8-bit floating point, FN variant): sign bit 7, exponent bits 6..3 (bias 7),
 * mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity. */
static double dec_e4m3(uint8_t code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp(m / 8.0, -6);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0 (OCP MX v1.0 scale): 2^(code - 127); code 255 is NaN. */
static double dec_e8m0(uint8_t code) { return code == 255 ? NAN : ldexp(1.0, (int)code - 127); }

/* Decoded values of every E2M1 and E4M3 code, filled once from the decoders above. */
static double g_e2m1[16], g_e4m3[256];
static int g_tables_ready = 0;

static void init_tables(void) {
    if (g_tables_ready) return;
    for (int c = 0; c < 16; ++c) g_e2m1[c] = dec_e2m1((uint8_t)c);
    for (int c = 0; c < 256; ++c) g_e4m3[c] = dec_e4m3((uint8_t)c);
    g_tables_ready = 1;
}

static float act_f(const void* p, int dt, int64_t i) {
    if (dt == ORC_F32) return ((const float*)p)[i];
    return dec_bf16_f(((const uint16_t*)p)[i]);
}

void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (double)dec_bf16_f(in[i]);
}
void oracle_decode_e2m1(const uint8_t* codes, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = dec_e2m1(codes[i] & 15);
}
void oracle_decode_e4m3(const uint8_t* codes, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = dec_e4m3(codes[i]);
}
void oracle_decode_e8m0(const uint8_t* codes, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = dec_e8m0(codes[i]);
}

/* Nearest E4M3 code of a magnitude a in [0, 448]; on a tie the code with the even mantissa
 * (even code) wins.  Binary search over the ascending positive codes 0..126. */
static uint8_t e4m3_nearest(double a) {
    int lo = 0, hi = 126; /* g_e4m3[lo] <= a <= g_e4m3[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_e4m3[mid] <= a) lo = mid; else hi = mid;
    }
    double dl = a - g_e4m3[lo], dh = g_e4m3[hi] - a;
    if (dl < dh) return (uint8_t)lo;
    if (dh < dl) return (uint8_t)hi;
    return (uint8_t)((lo & 1) ? hi : lo);
}

/* MX quantization of one block of 32 values (see the header): codes[32], the E8M0 scale code,
 * and the decoded values (what the quantized block stands for). */
static void mx_quantize_block(const double* v, uint8_t* codes, uint8_t* scale, double* dec) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[i]));
    int X = -127;
    if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* amax = m 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1 */
        X = ex - 1 - 8;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    *scale = (uint8_t)(X + 127);
    for (int i = 0; i < 32; ++i) {
        double q = fabs(ldexp(v[i], -X));
        if (q > 448.0) q = 448.0;
        uint8_t c = e4m3_nearest(q);
        int neg = signbit(v[i]) != 0;
        codes[i] = (uint8_t)(c | (neg ? 0x80 : 0));
        dec[i] = (neg ? -g_e4m3[c] : g_e4m3[c]) * ldexp(1.0, X);
    }
}

/* MX quantization of n blocks of 32 values each (v[n*32]): codes[n*32], scales[n], and the
 * decoded values dec[n*32] (any output may be NULL). */
void oracle_mx_quantize(const double* v, int64_t nblocks, uint8_t* codes, uint8_t* scales, double* dec) {
    init_tables();
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; ++b) {
        uint8_t c[32], s;
        double d[32];
        mx_quantize_block(v + b * 32, c, &s, d);
        if (codes) memcpy(codes + b * 32, c, 32);
        if (scales) scales[b] = s;
        if (dec) memcpy(dec + b * 32, d, sizeof d);
    }
}

/* Element (n, k) of one expert weight matrix with K columns, decoded to double. */
typedef struct {
    int dt;                 /* ORC_F32 | ORC_BF16 | ORC_NVFP4 */
    const void* w;          /* [rows, K] values, or packed nibbles [rows, K/2] */
    const uint8_t* scale;   /* NVFP4: E4M3 [rows, K/16]; MXFP8: E8M0 [rows, K/32] */
    double gscale;          /* NVFP4: per-expert fp32 second-level scale */
    int64_t K;
} wmat;

static double wget(const wmat* m, int64_t n, int64_t k) {
    if (m->dt == ORC_F32) return ((const float*)m->w)[n * m->K + k];
    if (m->dt == ORC_BF16) return (double)dec_bf16_f(((const uint16_t*)m->w)[n * m->K + k]);
    if (m->dt == ORC_MXFP8)
        return g_e4m3[((const uint8_t*)m->w)[n * m->K + k]] *
               ldexp(1.0, (int)m->scale[n * (m->K / 32) + k / 32] - 127);
    if (m->dt == ORC_MXFP4) {
        uint8_t byte = ((const uint8_t*)m->w)[n * (m->K / 2) + k / 2];
        uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15); /* even k in the low nibble */
        return g_e2m1[code] * ldexp(1.0, (int)m->scale[n * (m->K / 32) + k / 32] - 127);
    }
    {
        uint8_t byte = ((const uint8_t*)m->w)[n * (m->K / 2) + k / 2];
        uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15); /* even k in the low nibble */
        double s = g_e4m3[m->scale[n * (m->K / 16) + k / 16]];
        return g_e2m1[code] * s * m->gscale;
    }
}

/* ------------------------------------------------------------------------------------ */
/* route                                                                                  */
/* ------------------------------------------------------------------------------------ */

/* Canonical fp32 router logit.  The hidden vector is cut into chunks of 8 consecutive
 * elements; chunk c belongs to partial sum p = c mod 64.  Each of the 64 partials starts at
 * +0 and absorbs its chunks in ascending c, element by element, with one correctly rounded
 * fused multiply-add per element.  The 64 partials are then folded pairwise:
 * for off = 32,16,8,4,2,1: a[p] = a[p] + a[p+off] for p < off.  The bias, if any, is added
 * to a[0] last, in fp32.  Requires H % 8 == 0. */
float oracle_logit(const void* x_row, const void* w_row, int dt, int64_t H, int has_bias, float bias) {
    float a[64];
    for (int p = 0; p < 64; ++p) a[p] = 0.0f;
    for (int64_t c = 0; c < H / 8; ++c) {
        int p = (int)(c % 64);
        for (int i = 0; i < 8; ++i) {
            int64_t h = 8 * c + i;
            a[p] = fmaf(act_f(x_row, dt, h), act_f(w_row, dt, h), a[p]);
        }
    }
    for (int off = 32; off >= 1; off >>= 1)
        for (int p = 0; p < off; ++p) a[p] = a[p] + a[p + off];
    if (has_bias) a[0] = a[0] + bias;
    return a[0];
}

void oracle_router_logits(int64_t T, int64_t H, int64_t E, int dt, const void* x, const void* wr,
                          const float* bias, float* logits) {
    size_t es = (dt == ORC_F32) ? 4 : 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t e = 0; e < E; ++e)
            logits[t * E + e] = oracle_logit((const char*)x + (size_t)(t * H) * es,
                                             (const char*)wr + (size_t)(e * H) * es, dt, H,
                                             bias != NULL, bias ? bias[e] : 0.0f);
}

/* Top-k of one row of logits: (logit descending, expert ascending); stored in that order.
 * Weights: softmax over the selected logits (renorm = 1) or the full softmax value of each
 * selected expert (renorm = 0), in double. */
void oracle_select(int64_t T, int64_t E, int k, const float* logits, int renorm, int32_t* ids,
                   double* w) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: the lower index keeps ties */
            }
            taken[best] = 1;
            ids[t * k + j] = (int32_t)best;
        }
        free(taken);
        double top = (double)l[ids[t * k]];
        double z = 0.0;
        if (renorm) {
            for (int j = 0; j < k; ++j) z += exp((double)l[ids[t * k + j]] - top);
        } else {
            for (int64_t e = 0; e < E; ++e) z += exp((double)l[e] - top);
        }
        for (int j = 0; j < k; ++j) w[t * k + j] = exp((double)l[ids[t * k + j]] - top) / z;
    }
}

/* ------------------------------------------------------------------------------------ */
/* permute                                                                                */
/* ------------------------------------------------------------------------------------ */

void oracle_permute(int64_t T, int k, int64_t E, int64_t eb, int64_t ee, const int32_t* ids,
                    int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm) {
    int64_t A = T * k;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t a = 0; a < A; ++a)
        if (ids[a] >= eb && ids[a] < ee) counts[ids[a]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e) next[e] = offsets[e];
    for (int64_t a = 0; a < A; ++a) { /* row-major (t, j) order: stable */
        if (ids[a] < eb || ids[a] >= ee) { /* expert not held: not dispatched */
            inv_perm[a] = -1;
            continue;
        }
        int32_t pos = next[ids[a]]++;
        sorted_token[pos] = (int32_t)(a / k);
        inv_perm[a] = pos;
    }
    free(next);
}

/* ------------------------------------------------------------------------------------ */
/* expert FFN                                                                             */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    int64_t H, F;
    int wdt;
    const void *w13, *w2;                 /* per-expert base pointers are computed below */
    const uint8_t *w13_scale, *w2_scale;
    const float *w13_gscale, *w2_gscale;  /* nullable: 1.0 */
} experts_t;

static void expert_mats(const experts_t* ex, int64_t e, wmat* g13, wmat* g2) {
    int64_t H = ex->H, F = ex->F;
    g13->dt = g2->dt = ex->wdt;
    g13->K = H;
    g2->K = F;
    g13->w = g2->w = NULL;
    g13->scale = g2->scale = NULL;
    g13->gscale = g2->gscale = 1.0;
    if (ex->wdt == ORC_NVFP4) {
        if (ex->w13) g13->w = (const uint8_t*)ex->w13 + e * (2 * F) * (H / 2);
        g2->w = (const uint8_t*)ex->w2 + e * H * (F / 2);
        if (ex->w13_scale) g13->scale = ex->w13_scale + e * (2 * F) * (H / 16);
        g2->scale = ex->w2_scale + e * H * (F / 16);
        g13->gscale = ex->w13_gscale ? ex->w13_gscale[e] : 1.0;
        g2->gscale = ex->w2_gscale ? ex->w2_gscale[e] : 1.0;
    } else if (ex->wdt == ORC_MXFP4) {
        if (ex->w13) g13->w = (const uint8_t*)ex->w13 + e * (2 * F) * (H / 2);
        g2->w = (const uint8_t*)ex->w2 + e * H * (F / 2);
        if (ex->w13_scale) g13->scale = ex->w13_scale + e * (2 * F) * (H / 32);
        g2->scale = ex->w2_scale + e * H * (F / 32);
    } else if (ex->wdt == ORC_MXFP8) {
        if (ex->w13) g13->w = (const uint8_t*)ex->w13 + e * (2 * F) * H;
        g2->w = (const uint8_t*)ex->w2 + e * H * F;
        if (ex->w13_scale) g13->scale = ex->w13_scale + e * (2 * F) * (H / 32);
        g2->scale = ex->w2_scale + e * H * (F / 32);
    } else {
        size_t es = ex->wdt == ORC_F32 ? 4 : 2;
        if (ex->w13) g13->w = (const char*)ex->w13 + (size_t)(e * 2 * F * H) * es;
        g2->w = (const char*)ex->w2 + (size_t)(e * H * F) * es;
    }
}

/* v rounded to the nearest bf16 value (8 significant bits), ties to even; directly from
 * double (no intermediate float), bf16 subnormals on the grid 2^-133. */
static double round_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    frexp(v, &e); /* |v| = m 2^e, m in [0.5, 1) */
    int q = e - 8; /* quantum of 8 significant bits */
    if (q < -133) q = -133;
    return ldexp(nearbyint(ldexp(v, -q)), q); /* nearbyint: round to nearest even */
}

/* Replace v[0:n] by its MX-quantized value (MXFP8 layers quantize their activations). */
static void mx_requantize(double* v, int64_t n) {
    uint8_t c[32], s;
    for (int64_t b = 0; b < n / 32; ++b) mx_quantize_block(v + 32 * b, c, &s, v + 32 * b);
}

/* hid[0:F] = silu(W13[e][0:F] . x) * (W13[e][F:2F] . x), silu(g) = g / (1 + e^-g), in double.
 * (For MXFP8 the caller passes the MX-quantized x.) */
static void gate_up_row(const experts_t* ex, int64_t e, const double* x, double* hid) {
    wmat g13, g2;
    expert_mats(ex, e, &g13, &g2);
    int64_t H = ex->H, F = ex->F;
    for (int64_t f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            g += wget(&g13, f, h) * x[h];
            u += wget(&g13, F + f, h) * x[h];
        }
        hid[f] = g / (1.0 + exp(-g)) * u;
    }
}

/* y[0:H] = W2[e] . hid, in double (for MXFP8, W2[e] . MX(hid)). */
static void down_row(const experts_t* ex, int64_t e, const double* hid, double* y) {
    wmat g13, g2;
    expert_mats(ex, e, &g13, &g2);
    int64_t H = ex->H, F = ex->F;
    const double* h_in = hid;
    double* hq = NULL;
    if (ex->wdt == ORC_MXFP8 || ex->wdt == ORC_MXFP4) {
        hq = (double*)malloc(sizeof(double) * (size_t)F);
        for (int64_t f = 0; f < F; ++f) hq[f] = round_bf16(hid[f]); /* hid is a bf16 activation */
        mx_requantize(hq, F);
        h_in = hq;
    }
    for (int64_t h = 0; h < H; ++h) {
        double s = 0.0;
        for (int64_t f = 0; f < F; ++f) s += wget(&g2, h, f) * h_in[f];
        y[h] = s;
    }
    free(hq);
}

/* Expert FFN of a list of assignment rows: row r runs expert row_expert[r] on token
 * row_token[r]; out[r, 0:H] (double).  hid_out[r, 0:F] optional (NULL to skip). */
void oracle_expert_rows(int64_t H, int64_t F, int act_dt, int wdt, const void* x, const void* w13,
                        const void* w2, const uint8_t* w13_scale, const uint8_t* w2_scale,
                        const float* w13_gscale, const float* w2_gscale, int64_t nrows,
                        const int32_t* row_token, const int32_t* row_expert, double* out,
                        double* hid_out) {
    experts_t ex = {H, F, wdt, w13, w2, w13_scale, w2_scale, w13_gscale, w2_gscale};
    init_tables();
#pragma omp parallel
    {
        double* xr = (double*)malloc(sizeof(double) * (size_t)H);
        double* hid = (double*)malloc(sizeof(double) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t t = row_token[r];
            for (int64_t h = 0; h < H; ++h) xr[h] = (double)act_f(x, act_dt, t * H + h);
            if (wdt == ORC_MXFP8 || wdt == ORC_MXFP4) mx_requantize(xr, H);
            gate_up_row(&ex, row_expert[r], xr, hid);
            if (out) down_row(&ex, row_expert[r], hid, out + r * H);
            if (hid_out) memcpy(hid_out + r * F, hid, sizeof(double) * (size_t)F);
        }
        free(xr);
        free(hid);
    }
}

/* The down projection alone: out[r, 0:H] = W2[row_expert[r]] . hid[r, 0:F] (hid in double). */
void oracle_down_rows(int64_t H, int64_t F, int wdt, const void* w2, const uint8_t* w2_scale,
                      const float* w2_gscale, int64_t nrows, const int32_t* row_expert,
                      const double* hid, double* out) {
    experts_t ex = {H, F, wdt, NULL, w2, NULL, w2_scale, NULL, w2_gscale};
    init_tables();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) down_row(&ex, row_expert[r], hid + r * F, out + r * H);
}

/* ------------------------------------------------------------------------------------ */
/* combine                                                                                */
/* ------------------------------------------------------------------------------------ */

void oracle_combine(int64_t T, int k, int64_t H, const double* y_perm, const int32_t* inv_perm,
                    const double* w, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            double s = 0.0;
            for (int j = 0; j < k; ++j)
                if (inv_perm[t * k + j] >= 0) s += w[t * k + j] * y_perm[(int64_t)inv_perm[t * k + j] * H + h];
            y[t * H + h] = s;
        }
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
