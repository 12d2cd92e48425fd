/*
 * Drives every oracle function on small inputs, including the degenerate
 * ones (E = 1, k = E, one token, no drafted tokens, tokens outside the
 * vocabulary, NaN and negative entries, r outside [0, 1)), for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access,
 * leak or undefined operation in the oracle ends the run with an error.
 * Inputs come from a small xorshift generator (test data only).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (uint32_t)(st >> 11);
}
static float unif(void) { return (float)(rnd() & 0xFFFFFF) / 16777216.0f; }
static float gauss(void) {
    float s = 0.f;
    for (int i = 0; i < 12; ++i) s += unif();
    return s - 6.f;
}
static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static void* xcalloc(size_t n, size_t sz) {
    void* p = calloc(n ? n : 1, sz);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void codecs(void) {
    double acc = 0;
    for (uint32_t c = 0; c < 16; ++c) acc += orc_e2m1_value(c);
    for (uint32_t b = 0; b < 256; ++b) {
        const double v = orc_e8m0_value(b), w = orc_e4m3_value(b);
        if (!isnan(v)) acc += v * 1e-40;
        if (!isnan(w)) acc += w;
    }
    const double probes[] = {0.0, -0.0, 0.25, 0.75, 5.0, 6.5, 1e9, -1e9, 448.0, 464.0, 1e-9, -3.0};
    for (size_t i = 0; i < sizeof probes / sizeof probes[0]; ++i)
        acc += orc_e2m1_round(probes[i]) + orc_e4m3_round(probes[i]);
    if (acc == 12345.0) puts("");
}

static void quantisers(int64_t rows, int64_t K) {
    float* w = xcalloc((size_t)(rows * K), sizeof(float));
    double* v = xcalloc((size_t)(rows * K), sizeof(double));
    for (int64_t i = 0; i < rows * K; ++i) {
        w[i] = (i % 97 == 0) ? 0.f : gauss() * 0.02f;
        v[i] = gauss() * (i % 31 == 0 ? 1e5 : 1.0);
    }
    uint8_t* p = xcalloc((size_t)(rows * K / 2), 1);
    uint8_t* s = xcalloc((size_t)(rows * K / 32), 1);
    uint8_t* c = xcalloc((size_t)(rows * K), 1);
    double* out = xcalloc((size_t)(rows * K), sizeof(double));
    orc_quant_mxfp4(w, rows, K, p, s);
    orc_dequant_mxfp4(p, s, rows, K, out);
    orc_quant_mxfp8(v, rows, K, c, s);
    orc_dequant_mxfp8(c, s, rows, K, out);
    free(w); free(v); free(p); free(s); free(c); free(out);
}

static void router(int32_t T, int32_t d, int32_t E) {
    uint16_t* x = xcalloc((size_t)T * d, 2);
    uint16_t* w = xcalloc((size_t)E * d, 2);
    for (int64_t i = 0; i < (int64_t)T * d; ++i) x[i] = bf16(gauss());
    for (int64_t i = 0; i < (int64_t)E * d; ++i) w[i] = bf16(gauss() * 0.02f);
    double* lg = xcalloc((size_t)T * E, sizeof(double));
    double* ad = xcalloc((size_t)T * E, sizeof(double));
    orc_router_logits(x, w, T, d, E, lg, ad);
    orc_router_logits(x, w, T, d, E, lg, NULL);
    free(x); free(w); free(lg); free(ad);
}

static void layer(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k, int32_t mode, int ties) {
    uint16_t* x = xcalloc((size_t)T * d, 2);
    float* lg = xcalloc((size_t)T * E, sizeof(float));
    for (int64_t i = 0; i < (int64_t)T * d; ++i) x[i] = bf16(gauss());
    for (int64_t i = 0; i < (int64_t)T * E; ++i) lg[i] = ties ? (float)(rnd() % 3) : gauss();
    const int64_t gu = (int64_t)E * f * d, dn = (int64_t)E * d * f;
    float* wf = xcalloc((size_t)(gu > dn ? gu : dn), sizeof(float));
    uint8_t *g = xcalloc((size_t)gu / 2, 1), *gs = xcalloc((size_t)gu / 32, 1);
    uint8_t *u = xcalloc((size_t)gu / 2, 1), *us = xcalloc((size_t)gu / 32, 1);
    uint8_t *dw = xcalloc((size_t)dn / 2, 1), *ds = xcalloc((size_t)dn / 32, 1);
    for (int64_t i = 0; i < gu; ++i) wf[i] = gauss() * 0.02f;
    orc_quant_mxfp4(wf, (int64_t)E * f, d, g, gs);
    orc_quant_mxfp4(wf, (int64_t)E * f, d, u, us);
    orc_quant_mxfp4(wf, (int64_t)E * d, f, dw, ds);
    double* y = xcalloc((size_t)T * d, sizeof(double));
    int32_t* ids = xcalloc((size_t)T * k, sizeof(int32_t));
    double* tw = xcalloc((size_t)T * k, sizeof(double));
    double* h = xcalloc((size_t)T * k * f, sizeof(double));
    if (orc_moe_forward(T, d, f, E, k, mode, x, lg, g, gs, u, us, dw, ds, y, ids, tw, h, 1) < 0) {
        fprintf(stderr, "forward rejected a valid shape\n");
        exit(1);
    }
    orc_moe_forward(T, d, f, E, k, mode, x, lg, g, gs, u, us, dw, ds, y, NULL, NULL, NULL, 1);
    int32_t *cnt = xcalloc((size_t)E, sizeof(int32_t)), *off = xcalloc((size_t)E + 1, sizeof(int32_t));
    int32_t *srt = xcalloc((size_t)T * k, sizeof(int32_t)), *inv = xcalloc((size_t)T * k, sizeof(int32_t));
    orc_route(lg, T, E, k, ids, tw);
    orc_permute(ids, T, k, E, cnt, off, srt, inv);
    free(x); free(lg); free(wf); free(g); free(gs); free(u); free(us); free(dw); free(ds);
    free(y); free(ids); free(tw); free(h); free(cnt); free(off); free(srt); free(inv);
}

static void dflash(int32_t B, int32_t G, int32_t V, int junk) {
    int32_t* draft = xcalloc((size_t)B * G, sizeof(int32_t));
    float* pd = xcalloc((size_t)B * G * V, sizeof(float));
    float* pt = xcalloc((size_t)B * (G + 1) * V, sizeof(float));
    float* u = xcalloc((size_t)B * G, sizeof(float));
    float* r = xcalloc((size_t)B, sizeof(float));
    for (int64_t i = 0; i < (int64_t)B * G * V; ++i) pd[i] = unif() / V * 2.f;
    for (int64_t i = 0; i < (int64_t)B * (G + 1) * V; ++i) {
        pt[i] = unif() / V * 2.f;
        if (junk && i % 7 == 0) pt[i] = (i % 2) ? NAN : -1.f;
    }
    for (int64_t i = 0; i < (int64_t)B * G; ++i) {
        const uint32_t z = rnd();
        draft[i] = junk && z % 5 == 0 ? (z % 2 ? -1 : V + (int32_t)(z % 100)) : (int32_t)(z % (uint32_t)V);
        u[i] = unif();
    }
    const float rs[] = {0.f, 0.5f, 0.99999994f, 1.f, 2.f, -1.f, NAN, INFINITY};
    for (int32_t b = 0; b < B; ++b) r[b] = junk ? rs[b % 8] : unif();
    int32_t* n = xcalloc((size_t)B, sizeof(int32_t));
    int32_t* tok = xcalloc((size_t)B, sizeof(int32_t));
    orc_dflash_accept(B, G, V, draft, pd, pt, u, r, n, tok);
    for (int32_t b = 0; b < B; ++b)
        if (n[b] < 0 || n[b] > G || tok[b] < -1 || tok[b] >= V) {
            fprintf(stderr, "dflash result out of range\n");
            exit(1);
        }
    free(draft); free(pd); free(pt); free(u); free(r); free(n); free(tok);
}

int main(void) {
    codecs();
    quantisers(3, 64);
    quantisers(1, 32);
    router(5, 96, 3);
    router(1, 32, 1);
    layer(8, 256, 512, 4, 2, ORC_ACT_BF16, 0);
    layer(3, 64, 64, 1, 1, ORC_ACT_BF16, 0);        /* one expert */
    layer(5, 64, 96, 6, 6, ORC_ACT_MXFP8, 1);       /* k = E, tied logits */
    layer(1, 32, 32, 3, 2, ORC_ACT_MXFP8, 0);       /* one token */
    dflash(6, 4, 37, 0);
    dflash(16, 8, 64, 1);                           /* out-of-range tokens, NaN and negative entries, r ends */
    dflash(3, 0, 10, 0);                            /* no drafted tokens */
    dflash(2, 2, 1, 1);                             /* a one-entry vocabulary */
    puts("oracle sanitizer run: ok");
    return 0;
}
