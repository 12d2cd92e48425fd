/*
 * CPU oracle of the MXFP4 MoE expert FFN -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this code.  It shares no source with the GPU library.
 *
 * What the path computes, with the passages each step follows:
 *   - Expert weights are MXFP4: 4-bit E2M1 elements, one power-of-two E8M0
 *     scale per block of 32 elements along the reduction dimension
 *     (ai.appwright.xyz tag page "投機的デコード", section
 *     "第1層：FP4量子化（モデル側）"; techllm.github.io "Xiaomi MiMo x TileRT",
 *     section "1. MXFP4 — MoE에만 걸린 양자화").  Element/scale bit meanings
 *     and the scalar-to-MX conversion follow the OCP Microscaling Formats
 *     (MX) v1.0 specification, which the format name refers to.
 *   - Tokens are routed to experts (techllm, section "3. TileRT", which names
 *     the expert-routing communication pattern); the pages give no routing
 *     rule, so the reading taken is: top-k of the router logits, softmax over
 *     the k selected.
 *   - Each selected expert is a gated FFN; the pages name no activation, so
 *     the reading taken is SwiGLU: h = silu(W_gate a) * (W_up a),
 *     o = W_down h, y = sum_j w_j o_j.
 *
 * Arithmetic is double precision in natural loop order.  OpenMP is used only
 * across tokens, whose results are independent, so it cannot change them.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Codecs                                                                     */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes for the 3 low code bits: exponent bias 1, one mantissa
 * bit; exponent field 0 is the subnormal 0 / 0.5.  (OCP MX v1.0, FP4 E2M1.) */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(uint32_t nibble) {
    double m = E2M1_MAG[nibble & 7u];
    return (nibble & 8u) ? -m : m;
}

/* E8M0 scale: unsigned exponent, bias 127, no mantissa; 0xFF is NaN. */
double orc_e8m0_value(uint32_t byte) {
    byte &= 0xFFu;
    if (byte == 0xFFu) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* OCP E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448. */
double orc_e4m3_value(uint32_t byte) {
    uint32_t s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) mag = ldexp((double)m / 8.0, -6);          /* subnormal */
    else         mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Round |q| to the nearest of the n ascending non-negative grid values;
 * on an exact tie take the even code (the grid index is the magnitude code,
 * so "even" is round-half-to-even on the element's mantissa LSB).  Values
 * beyond the last grid point saturate to it. */
static uint32_t nearest_even_code(double a, const double* grid, int n) {
    int best = 0;
    double bd = fabs(a - grid[0]);
    for (int i = 1; i < n; ++i) {
        double dd = fabs(a - grid[i]);
        if (dd < bd || (dd == bd && (i & 1) == 0)) {
            best = i;
            bd = dd;
        }
    }
    return (uint32_t)best;
}

uint32_t orc_e2m1_round(double q) {
    uint32_t sign = signbit(q) ? 8u : 0u;          /* -0 keeps its sign */
    double a = fabs(q);
    if (a > 6.0) a = 6.0;
    return sign | nearest_even_code(a, E2M1_MAG, 8);
}

static double E4M3_GRID[127];                       /* codes 0x00..0x7E */
static int e4m3_grid_ready = 0;

static void e4m3_grid_init(void) {
    if (e4m3_grid_ready) return;
    for (int c = 0; c < 127; ++c) E4M3_GRID[c] = orc_e4m3_value((uint32_t)c);
    e4m3_grid_ready = 1;
}

uint32_t orc_e4m3_round(double q) {
    e4m3_grid_init();
    uint32_t sign = signbit(q) ? 0x80u : 0u;
    double a = fabs(q);
    if (a > 448.0) a = 448.0;
    return sign | nearest_even_code(a, E4M3_GRID, 127);
}

/* Shared scale exponent of one block (OCP MX v1.0 scalar-to-MX conversion):
 * X = 2^(floor(log2(amax)) - emax_elem), floor(log2) taken exactly from the
 * binary exponent, clamped to the E8M0 range [-127, 127].  An all-zero block
 * gets the smallest scale. */
static int block_scale_exp(double amax, int emax_elem) {
    if (amax == 0.0) return -127;
    int ex;
    (void)frexp(amax, &ex);            /* amax = m * 2^ex, m in [0.5, 1) */
    int se = (ex - 1) - emax_elem;
    if (se < -127) se = -127;
    if (se > 127) se = 127;
    return se;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 tensors                                                              */
/* ------------------------------------------------------------------------ */

void orc_dequant_mxfp4(const uint8_t* packed, const uint8_t* scales,
                       int64_t rows, int64_t K, double* out) {
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t kk = 0; kk < K; ++kk) {
            uint8_t byte = packed[r * (K / 2) + kk / 2];
            uint32_t nib = (kk % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
            double s = orc_e8m0_value(scales[r * (K / ORC_MX_BLOCK) + kk / ORC_MX_BLOCK]);
            out[r * K + kk] = orc_e2m1_value(nib) * s;
        }
    }
}

void orc_quant_mxfp4(const float* w, int64_t rows, int64_t K,
                     uint8_t* packed, uint8_t* scales) {
    const int64_t nb = K / ORC_MX_BLOCK;
    for (int64_t r = 0; r < rows; ++r) {
        memset(packed + r * (K / 2), 0, (size_t)(K / 2));
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = w + r * K + b * ORC_MX_BLOCK;
            double amax = 0.0;
            for (int i = 0; i < ORC_MX_BLOCK; ++i)
                if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
            int se = block_scale_exp(amax, 2);      /* emax of E2M1 is 2 */
            scales[r * nb + b] = (uint8_t)(se + 127);
            for (int i = 0; i < ORC_MX_BLOCK; ++i) {
                int64_t kk = b * ORC_MX_BLOCK + i;
                uint32_t code = orc_e2m1_round(ldexp((double)v[i], -se));
                packed[r * (K / 2) + kk / 2] |= (uint8_t)((kk % 2 == 0) ? code : (code << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP8 (E4M3) tensors                                                       */
/* ------------------------------------------------------------------------ */

void orc_quant_mxfp8(const double* v, int64_t rows, int64_t K,
                     uint8_t* codes, uint8_t* scales) {
    const int64_t nb = K / ORC_MX_BLOCK;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const double* p = v + r * K + b * ORC_MX_BLOCK;
            double amax = 0.0;
            for (int i = 0; i < ORC_MX_BLOCK; ++i)
                if (fabs(p[i]) > amax) amax = fabs(p[i]);
            int se = block_scale_exp(amax, 8);      /* emax of E4M3 is 8 */
            scales[r * nb + b] = (uint8_t)(se + 127);
            for (int i = 0; i < ORC_MX_BLOCK; ++i)
                codes[r * K + b * ORC_MX_BLOCK + i] = (uint8_t)orc_e4m3_round(ldexp(p[i], -se));
        }
    }
}

void orc_dequant_mxfp8(const uint8_t* codes, const uint8_t* scales,
                       int64_t rows, int64_t K, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t kk = 0; kk < K; ++kk)
            out[r * K + kk] = orc_e4m3_value(codes[r * K + kk]) *
                              orc_e8m0_value(scales[r * (K / ORC_MX_BLOCK) + kk / ORC_MX_BLOCK]);
}

/* ------------------------------------------------------------------------ */
/* Routing and permutation                                                    */
/* ------------------------------------------------------------------------ */

/* One token: the k largest logits, in order of descending logit and, on
 * equal logits, ascending expert index; weights are the softmax over the k
 * selected logits. */
static void route_one(const float* l, int32_t E, int32_t k,
                      int32_t* ids, double* w, unsigned char* taken) {
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e)
            if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
        ids[j] = best;
        taken[best] = 1;
    }
    double l0 = (double)l[ids[0]], sum = 0.0;
    for (int32_t j = 0; j < k; ++j) sum += exp((double)l[ids[j]] - l0);
    for (int32_t j = 0; j < k; ++j) w[j] = exp((double)l[ids[j]] - l0) / sum;
}

void orc_route(const float* logits, int32_t T, int32_t E, int32_t k,
               int32_t* topk_ids, double* topk_w) {
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    for (int32_t t = 0; t < T; ++t)
        route_one(logits + (int64_t)t * E, E, k, topk_ids + (int64_t)t * k,
                  topk_w + (int64_t)t * k, taken);
    free(taken);
}

/* Pairs p = t*k + j grouped by expert: a counting sort that visits p in
 * ascending order, so pairs of one expert stay in ascending p. */
void orc_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                 int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                 int32_t* inverse) {
    const int32_t P = T * k;
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int32_t p = 0; p < P; ++p) counts[topk_ids[p]] += 1;
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int32_t p = 0; p < P; ++p) {
        int32_t pos = cursor[topk_ids[p]]++;
        sorted_pairs[pos] = p;
        inverse[p] = pos;
    }
    free(cursor);
}

/* ------------------------------------------------------------------------ */
/* DFlash verify acceptance                                                   */
/* ------------------------------------------------------------------------ */

/* Integer weight of one entry: rint(2^32 w) for w > 0; zero for w <= 0 and
 * for NaN (entries outside a probability's range carry no mass). */
static uint64_t int_weight(float w) {
    return w > 0.0f ? (uint64_t)rint((double)w * 4294967296.0) : 0;
}

/* Index drawn from weights w[0..V) with the uniform r: integer weights
 * q_i = int_weight(w_i), S = sum q_i, threshold = floor(S * r24 / 2^24) with
 * r24 = floor(2^24 r) clamped to [0, 2^24 - 1] (r below 0 or NaN counts as
 * 0, r at or above 1 as the largest float below 1), result = the first i
 * whose inclusive prefix sum of q exceeds the threshold.  Integer sums make
 * the draw independent of summation order.  Returns -1 when S == 0. */
static int32_t draw_index(const float* w, int32_t V, float r) {
    uint64_t S = 0;
    for (int32_t i = 0; i < V; ++i) S += int_weight(w[i]);
    if (S == 0) return -1;
    uint64_t r24 = 0;
    if (r > 0.0f) {
        const double f = floor((double)r * 16777216.0);
        r24 = f >= 16777215.0 ? 16777215u : (uint64_t)f;
    }
    const uint64_t thr = (uint64_t)(((unsigned __int128)S * r24) >> 24);
    uint64_t run = 0;
    for (int32_t i = 0; i < V; ++i) {
        run += int_weight(w[i]);
        if (run > thr) return i;
    }
    return -1;                                      /* not reached: thr < S */
}

/* The pages make the verification of a drafted block lossless with a final
 * rejection-sampling pass (techllm.github.io "Xiaomi MiMo x TileRT", section
 * "2. DFlash") without printing the rule; the reading is standard
 * speculative sampling.  Position j's draft token x is accepted when
 * u_j * p_draft[j][x] < p_target[j][x] (u_j < p_target / p_draft, decided
 * in float32); the first rejection ends the block and the next token is
 * drawn from max(0, p_target[j] - p_draft[j]) (float32 per element), or from
 * p_target[j] if that residual rounds to nothing; after G acceptances it is
 * drawn from p_target[G].  A draft token outside [0, V) is rejected (it has
 * no probability to compare). */
void orc_dflash_accept(int32_t B, int32_t G, int32_t V, const int32_t* draft, const float* p_draft,
                       const float* p_target, const float* u, const float* r, int32_t* n_accepted,
                       int32_t* next_token) {
    float* res = (float*)malloc(sizeof(float) * (size_t)(V > 0 ? V : 1));
    for (int32_t b = 0; b < B; ++b) {
        int32_t j = 0;
        for (; j < G; ++j) {
            const int32_t x = draft[(int64_t)b * G + j];
            if (x < 0 || x >= V) break;
            const float pd = p_draft[((int64_t)b * G + j) * V + x];
            const float pt = p_target[((int64_t)b * (G + 1) + j) * V + x];
            const float up = u[(int64_t)b * G + j] * pd;
            if (!(up < pt)) break;
        }
        n_accepted[b] = j;
        const float* pt_row = p_target + ((int64_t)b * (G + 1) + j) * V;
        int32_t tok = -1;
        if (j < G) {
            const float* pd_row = p_draft + ((int64_t)b * G + j) * V;
            for (int32_t i = 0; i < V; ++i) {
                const float dlt = pt_row[i] - pd_row[i];
                res[i] = dlt > 0.0f ? dlt : 0.0f;
            }
            tok = draw_index(res, V, r[b]);
        }
        if (tok < 0) tok = draw_index(pt_row, V, r[b]);
        next_token[b] = tok;
    }
    free(res);
}

/* ------------------------------------------------------------------------ */
/* Expert layer                                                               */
/* ------------------------------------------------------------------------ */

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Router projection that produces the routing logits from the hidden
 * states.  The pages keep every module outside the experts in FP8 or its
 * original precision (techllm.github.io "Xiaomi MiMo x TileRT", section
 * "1. MXFP4 — MoE에만 걸린 양자화") and route each token to its experts
 * (same page, section "3. TileRT"), but give no router form; the reading
 * taken is the plain linear map logits = x W^T with bf16 x and W and no
 * bias.  Every product of two bf16 values is exact in double; the sum is
 * taken in index order. */
void orc_router_logits(const uint16_t* x_bf16, const uint16_t* w_bf16, int32_t T, int32_t d,
                       int32_t E, double* logits, double* absdot) {
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t* xt = x_bf16 + (int64_t)t * d;
        for (int32_t e = 0; e < E; ++e) {
            const uint16_t* we = w_bf16 + (int64_t)e * d;
            double s = 0.0, a = 0.0;
            for (int32_t i = 0; i < d; ++i) {
                const double p = bf16_value(xt[i]) * bf16_value(we[i]);
                s += p;
                a += fabs(p);
            }
            logits[(int64_t)t * E + e] = s;
            if (absdot) absdot[(int64_t)t * E + e] = a;
        }
    }
}

/* Element [r][kk] of an MXFP4 matrix with K columns. */
static double w_elem(const uint8_t* packed, const uint8_t* scales, int64_t K,
                     int64_t r, int64_t kk) {
    uint8_t byte = packed[r * (K / 2) + kk / 2];
    uint32_t nib = (kk % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
    return orc_e2m1_value(nib) *
           orc_e8m0_value(scales[r * (K / ORC_MX_BLOCK) + kk / ORC_MX_BLOCK]);
}

/* In-place MXFP8 round trip of one vector of length K (K % 32 == 0). */
static void mxfp8_round_trip(double* v, int64_t K, uint8_t* codes, uint8_t* scales) {
    orc_quant_mxfp8(v, 1, K, codes, scales);
    orc_dequant_mxfp8(codes, scales, 1, K, v);
}

int32_t orc_moe_forward(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                        int32_t act_mode, const uint16_t* x_bf16,
                        const float* logits,
                        const uint8_t* w_gate, const uint8_t* w_gate_scale,
                        const uint8_t* w_up, const uint8_t* w_up_scale,
                        const uint8_t* w_down, const uint8_t* w_down_scale,
                        double* y, int32_t* topk_ids, double* topk_w,
                        double* h, int32_t nthreads) {
    if (T < 0 || d <= 0 || f <= 0 || E <= 0 || k <= 0 || k > E ||
        d % ORC_MX_BLOCK || f % ORC_MX_BLOCK ||
        (act_mode != ORC_ACT_BF16 && act_mode != ORC_ACT_MXFP8))
        return -1;
    e4m3_grid_init();
    const int64_t gate_sz = (int64_t)f * d / 2, gate_sc = (int64_t)f * d / ORC_MX_BLOCK;
    const int64_t down_sz = (int64_t)d * f / 2, down_sc = (int64_t)d * f / ORC_MX_BLOCK;
    int32_t used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* a = (double*)malloc(sizeof(double) * (size_t)d);
        double* g = (double*)malloc(sizeof(double) * (size_t)f);
        double* u = (double*)malloc(sizeof(double) * (size_t)f);
        double* hh = (double*)malloc(sizeof(double) * (size_t)f);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        uint8_t* qc = (uint8_t*)malloc((size_t)(d > f ? d : f));
        uint8_t* qs = (uint8_t*)malloc((size_t)(d > f ? d : f) / ORC_MX_BLOCK + 1);
        int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        double* wt = (double*)malloc(sizeof(double) * (size_t)k);
        unsigned char* taken = (unsigned char*)malloc((size_t)E);

#pragma omp for schedule(dynamic, 1)
        for (int32_t t = 0; t < T; ++t) {
            /* activations: bf16 widened exactly, optionally MXFP8 round trip */
            for (int32_t i = 0; i < d; ++i) a[i] = bf16_value(x_bf16[(int64_t)t * d + i]);
            if (act_mode == ORC_ACT_MXFP8) mxfp8_round_trip(a, d, qc, qs);

            route_one(logits + (int64_t)t * E, E, k, ids, wt, taken);
            if (topk_ids) for (int32_t j = 0; j < k; ++j) topk_ids[(int64_t)t * k + j] = ids[j];
            if (topk_w) for (int32_t j = 0; j < k; ++j) topk_w[(int64_t)t * k + j] = wt[j];

            double* yt = y + (int64_t)t * d;
            for (int32_t m = 0; m < d; ++m) yt[m] = 0.0;

            for (int32_t j = 0; j < k; ++j) {
                const int64_t e = ids[j];
                const uint8_t *gp = w_gate + e * gate_sz, *gs = w_gate_scale + e * gate_sc;
                const uint8_t *up = w_up + e * gate_sz, *us = w_up_scale + e * gate_sc;
                const uint8_t *dp = w_down + e * down_sz, *ds = w_down_scale + e * down_sc;
                /* gate / up projections and SwiGLU */
                for (int32_t n = 0; n < f; ++n) {
                    double gn = 0.0, un = 0.0;
                    for (int32_t kk = 0; kk < d; ++kk) {
                        gn += w_elem(gp, gs, d, n, kk) * a[kk];
                        un += w_elem(up, us, d, n, kk) * a[kk];
                    }
                    g[n] = gn;
                    u[n] = un;
                    hh[n] = gn / (1.0 + exp(-gn)) * un;
                }
                if (act_mode == ORC_ACT_MXFP8) mxfp8_round_trip(hh, f, qc, qs);
                if (h) memcpy(h + ((int64_t)t * k + j) * f, hh, sizeof(double) * (size_t)f);
                /* down projection and weighted combine */
                for (int32_t m = 0; m < d; ++m) {
                    double om = 0.0;
                    for (int32_t n = 0; n < f; ++n) om += w_elem(dp, ds, f, m, n) * hh[n];
                    o[m] = om;
                }
                for (int32_t m = 0; m < d; ++m) yt[m] += wt[j] * o[m];
            }
        }
        free(a); free(g); free(u); free(hh); free(o); free(qc); free(qs);
        free(ids); free(wt); free(taken);
    }
    return used;
}
