/*
 * sanitize_driver.c -- runs every entry point of attn_oracle.c on small
 * seeded inputs, edge cases included (no keys, no valid query, one token, a
 * row subset, query offset with a key range of its own, window 1, extent 1,
 * bf16 profiles, flex masks with and without sinks), so that the oracle can
 * be built and exercised under AddressSanitizer and UndefinedBehaviorSanitizer
 * on the CPU.  Test infrastructure only, like the oracle itself.  Exit status 0
 * when every call returned 0 and every result is finite where it must be.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int attn_oracle_fwd(const uint16_t*, const uint16_t*, const uint16_t*, const void*, int, const float*,
                    const uint8_t*, const uint8_t*, const int32_t*, const int32_t*, int64_t, int64_t, int, int,
                    int, int, int, int, int, const int64_t*, int64_t, double*, double*, int32_t*, int);
int flex_oracle_fwd(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const int32_t*, int32_t,
                    int64_t, int64_t, double, int, int, int, int, int, int, const int64_t*, int64_t, double*,
                    double*, int32_t*, int);
int attn_oracle_bwd(const uint16_t*, const uint16_t*, const uint16_t*, const void*, int, const float*,
                    const uint8_t*, const uint8_t*, const int32_t*, const int32_t*, int64_t, int64_t, int, int,
                    int, int, int, int, int, const double*, const double*, int, int, int, double*, double*,
                    double*, double*, double*, int);
int attn_oracle_mask(const uint8_t*, const uint8_t*, const int32_t*, const int32_t*, int64_t, int64_t, int, int,
                     int, int32_t*, uint8_t*, int);

static uint64_t rng = 88172645463325252ull;
static double unif(void)   /* xorshift64 in [0, 1) */
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static uint16_t bf16_of(double x)   /* truncation is enough for test data */
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}
static void* xmalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) exit(3); return p; }

static int failures = 0;
static void expect(int ok, const char* what)
{
    if (!ok) { fprintf(stderr, "FAIL: %s\n", what); ++failures; }
}

/* One forward / backward / mask case: Sq queries at offset qoff against Sk keys.  Token t
   (global column) is not real when t % invalid_every == 1; invalid_every < 0: no token is. */
static void run_case(int B, int Sq, int Sk, int Hq, int Hkv, int D, int E, int64_t window, int64_t qoff,
                     int bf16_prof, int invalid_every, int doc_len, int use_rows)
{
    size_t nq = (size_t)B * Sq * Hq * D, nk = (size_t)B * Sk * Hkv * D, np_ = (size_t)B * Hq * Sq * E;
    uint16_t* q = xmalloc(nq * 2); uint16_t* k = xmalloc(nk * 2); uint16_t* v = xmalloc(nk * 2);
    float* pf = xmalloc(np_ * 4); uint16_t* pb = xmalloc(np_ * 2);
    float* sink = xmalloc((size_t)B * Sq * Hq * 4);
    uint8_t* valid = xmalloc((size_t)B * Sq); uint8_t* kvalid = xmalloc((size_t)B * Sk);
    int32_t* pos = xmalloc((size_t)B * Sq * 4); int32_t* kpos = xmalloc((size_t)B * Sk * 4);
    for (size_t t = 0; t < nq; ++t) q[t] = bf16_of(unif() * 2 - 1);
    for (size_t t = 0; t < nk; ++t) { k[t] = bf16_of(unif() * 2 - 1); v[t] = bf16_of(unif() * 2 - 1); }
    for (size_t t = 0; t < np_; ++t) { pf[t] = (float)(unif() - 0.5); pb[t] = bf16_of(pf[t]); }
    for (size_t t = 0; t < (size_t)B * Sq * Hq; ++t) sink[t] = (t % 5 == 0) ? -INFINITY : (float)(unif() * 4 - 2);
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < Sk; ++j) {
            kvalid[(size_t)b * Sk + j] = invalid_every < 0 ? 0 : invalid_every ? (j % invalid_every != 1) : 1;
            kpos[(size_t)b * Sk + j] = doc_len ? j % doc_len : j;
        }
        for (int i = 0; i < Sq; ++i) {
            int gi = (int)qoff + i;
            valid[(size_t)b * Sq + i] = invalid_every < 0 ? 0 : invalid_every ? (gi % invalid_every != 1) : 1;
            pos[(size_t)b * Sq + i] = doc_len ? gi % doc_len : gi;
        }
    }
    int64_t nrows = (int64_t)B * Sq;
    int64_t* rows = NULL;
    if (use_rows && nrows > 0) {
        nrows = nrows > 3 ? 3 : nrows;
        rows = xmalloc((size_t)nrows * 8);
        for (int64_t t = 0; t < nrows; ++t) rows[t] = ((int64_t)B * Sq - 1) - 2 * t > 0 ? ((int64_t)B * Sq - 1) - 2 * t : 0;
    }
    double* out = xmalloc((size_t)(nrows > 0 ? nrows : 1) * Hq * D * 8);
    double* lse = xmalloc((size_t)(nrows > 0 ? nrows : 1) * Hq * 8);
    int32_t* cnt = xmalloc((size_t)(nrows > 0 ? nrows : 1) * 4);
    expect(attn_oracle_fwd(q, k, v, bf16_prof ? (const void*)pb : (const void*)pf, bf16_prof, sink, valid, kvalid,
                           pos, kpos, window, qoff, B, Sq, Sk, Hq, Hkv, D, E, rows, nrows, out, lse, cnt, 2) == 0,
           "attn_oracle_fwd");
    for (int64_t t = 0; t < nrows * Hq * D; ++t) expect(isfinite(out[t]), "finite out");

    int32_t* cnt2 = xmalloc((size_t)B * Sq * 4 + 4);
    uint8_t* m = xmalloc((size_t)B * Sq * Sk + 1);
    expect(attn_oracle_mask(valid, kvalid, pos, kpos, window, qoff, B, Sq, Sk, cnt2, m, 2) == 0, "attn_oracle_mask");

    double* dout = xmalloc(nq * 8 + 8); double* dlse = xmalloc((size_t)B * Sq * Hq * 8 + 8);
    for (size_t t = 0; t < nq; ++t) dout[t] = unif() - 0.5;
    for (size_t t = 0; t < (size_t)B * Sq * Hq; ++t) dlse[t] = unif() - 0.5;
    double* dq = xmalloc(nq * 8 + 8); double* dk = xmalloc(nk * 8 + 8); double* dv = xmalloc(nk * 8 + 8);
    double* dp = xmalloc(np_ * 8 + 8); double* ds = xmalloc((size_t)B * Sq * Hq * 8 + 8);
    for (int mag = 0; mag < 2; ++mag)
        expect(attn_oracle_bwd(q, k, v, bf16_prof ? (const void*)pb : (const void*)pf, bf16_prof, sink, valid,
                               kvalid, pos, kpos, window, qoff, B, Sq, Sk, Hq, Hkv, D, E, dout,
                               mag ? NULL : dlse, Sq / 3, mag ? 0 : Sq - 2, mag, dq, dk, dv, dp, ds,
                               mag ? 1 : 3) == 0,
               "attn_oracle_bwd");
    free(q); free(k); free(v); free(pf); free(pb); free(sink); free(valid); free(kvalid); free(pos); free(kpos);
    free(rows); free(out); free(lse); free(cnt); free(cnt2); free(m); free(dout); free(dlse);
    free(dq); free(dk); free(dv); free(dp); free(ds);
}

static void run_flex(int B, int Sq, int Sk, int Hq, int Hkv, int D, int with_sink, int with_tokens, int64_t F,
                     int64_t W, int use_rows)
{
    size_t nq = (size_t)B * Hq * Sq * D, nk = (size_t)B * Hkv * Sk * D;
    uint16_t* q = xmalloc(nq * 2); uint16_t* k = xmalloc(nk * 2); uint16_t* v = xmalloc(nk * 2);
    float* sw = xmalloc((size_t)Hq * 4); int32_t* tok = xmalloc((size_t)B * Sq * 4 + 4);
    for (size_t t = 0; t < nq; ++t) q[t] = bf16_of(unif() * 2 - 1);
    for (size_t t = 0; t < nk; ++t) { k[t] = bf16_of(unif() * 2 - 1); v[t] = bf16_of(unif() * 2 - 1); }
    for (int h = 0; h < Hq; ++h) sw[h] = (float)(unif() * 2 - 1);
    for (size_t t = 0; t < (size_t)B * Sq; ++t) tok[t] = (int32_t)(unif() * 5);
    int64_t nrows = use_rows ? 2 : (int64_t)B * Sq;
    int64_t rows[2] = {0, (int64_t)B * Sq - 1};
    double* out = xmalloc((size_t)(nrows > 0 ? nrows : 1) * Hq * D * 8);
    double* lse = xmalloc((size_t)(nrows > 0 ? nrows : 1) * Hq * 8);
    int32_t* cnt = xmalloc((size_t)(nrows > 0 ? nrows : 1) * 4);
    expect(flex_oracle_fwd(q, k, v, with_sink ? sw : NULL, with_tokens ? tok : NULL, 0, F, W, 0.25, B, Sq, Sk, Hq,
                           Hkv, D, use_rows ? rows : NULL, nrows, out, lse, cnt, 2) == 0,
           "flex_oracle_fwd");
    free(q); free(k); free(v); free(sw); free(tok); free(out); free(lse); free(cnt);
}

int main(void)
{
    run_case(2, 37, 37, 4, 2, 8, 6, 0, 0, 0, 0, 0, 0);       /* causal, all valid */
    run_case(1, 40, 40, 6, 2, 16, 50, 5, 0, 1, 7, 11, 0);    /* window, holes, documents, bf16, E > S */
    run_case(2, 23, 51, 4, 4, 8, 1, 1, 28, 0, 4, 9, 1);      /* query offset, Sk != Sq, E = 1, W = 1, rows */
    run_case(1, 5, 0, 2, 1, 8, 3, 0, 9, 0, 0, 0, 0);         /* no keys */
    run_case(1, 1, 1, 2, 2, 4, 2, 0, 0, 0, 0, 0, 0);         /* one token */
    run_case(1, 30, 30, 2, 1, 8, 4, 0, 0, 1, -1, 0, 1);      /* no valid token at all */
    run_flex(2, 33, 33, 4, 2, 8, 1, 1, 0, 0, 0);
    run_flex(1, 40, 40, 4, 1, 16, 0, 0, 8, 5, 1);
    run_flex(1, 20, 35, 2, 2, 8, 1, 0, 0, 3, 0);
    if (failures) { fprintf(stderr, "%d failures\n", failures); return 1; }
    printf("sanitized oracle: all calls ok\n");
    return 0;
}
