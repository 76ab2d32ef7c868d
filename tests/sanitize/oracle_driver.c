/* Runs every entry point of the CPU oracle on small seeded shapes (fp32, bf16 and NVFP4
 * weights, k = E, E = 1, T = 0) so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer can check its memory accesses and arithmetic.  Exit status 0
 * when the structural invariants hold (weights sum to 1, the permutation is a bijection that
 * returns each assignment to its token, outputs are finite). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_router_logits(int64_t T, int64_t H, int64_t E, int dt, const void* x, const void* wr,
                          const float* bias, float* logits);
void oracle_select(int64_t T, int64_t E, int k, const float* logits, int renorm, int32_t* ids,
                   double* w);
void oracle_permute(int64_t T, int k, int64_t E, int64_t eb, int64_t ee, const int32_t* ids,
                    int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm);
void oracle_expert_rows(int64_t H, int64_t F, int act_dt, int wdt, const void* x, const void* w13,
                        const void* w2, const uint8_t* w13_scale, const uint8_t* w2_scale,
                        const float* w13_gscale, const float* w2_gscale, int64_t nrows,
                        const int32_t* row_token, const int32_t* row_expert, double* out,
                        double* hid_out);
void oracle_combine(int64_t T, int k, int64_t H, const double* y_perm, const int32_t* inv_perm,
                    const double* w, double* y);

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}
static float next_f(float scale) { return scale * ((float)(next_u32() % 2001u) / 1000.0f - 1.0f); }

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* act: 0 fp32, 1 bf16; wdt: 0 fp32, 1 bf16, 2 NVFP4 (bf16 activations) */
static int run_case(int T, int H, int E, int k, int F, int act, int wdt, int renorm) {
    const size_t ae = act ? 2 : 4;
    const int A = T * k;
    void* x = malloc((size_t)T * H * ae + 1);
    void* wr = malloc((size_t)E * H * ae);
    float* bias = malloc(sizeof(float) * (size_t)E);
    for (int64_t i = 0; i < (int64_t)T * H; ++i) {
        float v = next_f(1.0f);
        if (act) ((uint16_t*)x)[i] = to_bf16(v); else ((float*)x)[i] = v;
    }
    for (int64_t i = 0; i < (int64_t)E * H; ++i) {
        float v = next_f(0.05f);
        if (act) ((uint16_t*)wr)[i] = to_bf16(v); else ((float*)wr)[i] = v;
    }
    for (int e = 0; e < E; ++e) bias[e] = next_f(0.5f);
    size_t n13 = (size_t)E * 2 * F * H, n2 = (size_t)E * H * F;
    void *w13, *w2;
    uint8_t *s13 = NULL, *s2 = NULL;
    float *g13 = NULL, *g2 = NULL;
    if (wdt == 2) {
        w13 = malloc(n13 / 2);
        w2 = malloc(n2 / 2);
        for (size_t i = 0; i < n13 / 2; ++i) ((uint8_t*)w13)[i] = (uint8_t)next_u32();
        for (size_t i = 0; i < n2 / 2; ++i) ((uint8_t*)w2)[i] = (uint8_t)next_u32();
        s13 = malloc(n13 / 16);
        s2 = malloc(n2 / 16);
        for (size_t i = 0; i < n13 / 16; ++i) s13[i] = (uint8_t)(0x28 + next_u32() % 24);
        for (size_t i = 0; i < n2 / 16; ++i) s2[i] = (uint8_t)(0x28 + next_u32() % 24);
        g13 = malloc(sizeof(float) * (size_t)E);
        g2 = malloc(sizeof(float) * (size_t)E);
        for (int e = 0; e < E; ++e) g13[e] = g2[e] = 0.01f;
    } else {
        size_t we = wdt ? 2 : 4;
        w13 = malloc(n13 * we);
        w2 = malloc(n2 * we);
        for (size_t i = 0; i < n13; ++i) {
            float v = next_f(0.05f);
            if (wdt) ((uint16_t*)w13)[i] = to_bf16(v); else ((float*)w13)[i] = v;
        }
        for (size_t i = 0; i < n2; ++i) {
            float v = next_f(0.05f);
            if (wdt) ((uint16_t*)w2)[i] = to_bf16(v); else ((float*)w2)[i] = v;
        }
    }
    float* logits = malloc(sizeof(float) * ((size_t)T * E + 1));
    int32_t* ids = malloc(sizeof(int32_t) * ((size_t)A + 1));
    double* w = malloc(sizeof(double) * ((size_t)A + 1));
    int32_t* counts = malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t* st = malloc(sizeof(int32_t) * ((size_t)A + 1));
    int32_t* ip = malloc(sizeof(int32_t) * ((size_t)A + 1));
    int32_t* rexp = malloc(sizeof(int32_t) * ((size_t)A + 1));
    double* yperm = malloc(sizeof(double) * ((size_t)A * H + 1));
    double* hid = malloc(sizeof(double) * ((size_t)A * F + 1));
    double* y = malloc(sizeof(double) * ((size_t)T * H + 1));
    int bad = 0;

    oracle_router_logits(T, H, E, act, x, wr, bias, logits);
    oracle_select(T, E, k, logits, renorm, ids, w);
    oracle_permute(T, k, E, 0, E, ids, counts, offsets, st, ip);
    for (int e = 0; e < E; ++e)
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) rexp[r] = e;
    oracle_expert_rows(H, F, act, wdt, x, w13, w2, s13, s2, g13, g2, A, st, rexp, yperm, hid);
    oracle_combine(T, k, H, yperm, ip, w, y);

    if (offsets[E] != A) bad = 1;
    for (int t = 0; t < T; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += w[t * k + j];
        if (renorm && fabs(s - 1.0) > 1e-12) bad = 1;
    }
    for (int a = 0; a < A; ++a) {
        if (ip[a] < 0 || ip[a] >= A || st[ip[a]] != a / k) bad = 1;
    }
    for (int64_t i = 0; i < (int64_t)T * H; ++i)
        if (!isfinite(y[i])) bad = 1;
    /* a held expert range (expert parallelism): upper half of the experts */
    {
        const int eb = E / 2;
        oracle_permute(T, k, E, eb, E, ids, counts, offsets, st, ip);
        int held = 0;
        for (int a = 0; a < A; ++a) {
            const int in = ids[a] >= eb;
            held += in;
            if (in ? (ip[a] < 0 || ip[a] >= offsets[E] || st[ip[a]] != a / k) : ip[a] != -1) bad = 1;
        }
        if (offsets[E] != held) bad = 1;
        oracle_combine(T, k, H, yperm, ip, w, y);
        for (int64_t i = 0; i < (int64_t)T * H; ++i)
            if (!isfinite(y[i])) bad = 1;
    }
    printf("case T=%d H=%d E=%d k=%d F=%d act=%d wdt=%d renorm=%d: %s\n", T, H, E, k, F, act, wdt,
           renorm, bad ? "FAILED" : "ok");

    free(x); free(wr); free(bias); free(w13); free(w2); free(s13); free(s2); free(g13); free(g2);
    free(logits); free(ids); free(w); free(counts); free(offsets); free(st); free(ip); free(rexp);
    free(yperm); free(hid); free(y);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run_case(5, 64, 8, 2, 64, 0, 0, 1);
    bad |= run_case(7, 64, 4, 4, 32, 1, 1, 1);   /* k = E */
    bad |= run_case(6, 64, 6, 2, 64, 1, 2, 1);   /* NVFP4 */
    bad |= run_case(3, 32, 1, 1, 16, 0, 0, 1);   /* one expert */
    bad |= run_case(4, 64, 8, 3, 32, 1, 1, 0);   /* full-softmax weights */
    bad |= run_case(0, 64, 8, 2, 64, 1, 1, 1);   /* no tokens */
    return bad;
}
