/*
 * CPU oracle of the MXFP4 MoE expert FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it includes nothing of the GPU library.
 *
 * Plain, slow, obviously-correct definitions in double precision.  Every
 * function names the passage it follows.  Sources:
 *   - ai.appwright.xyz, tag page "投機的デコード", article section
 *     "第1層：FP4量子化（モデル側）": MoE experts only are MXFP4 with a block
 *     size of 32 (one shared scale per 32 elements).
 *   - techllm.github.io, "Xiaomi MiMo x TileRT: 1T parameters at 1000+
 *     tokens/s", section "1. MXFP4 — MoE에만 걸린 양자화": FP4 is applied to
 *     the expert weights, which hold most of the parameters.
 *   - the same page, section "3. TileRT": tokens are routed to their experts
 *     (the router form and the top-k rule are readings, stated where used).
 *   - the same page, section "2. DFlash": a drafted block is verified by the
 *     target model, with a final rejection-sampling pass that keeps the
 *     output distribution the target's (the acceptance rule is the standard
 *     speculative-sampling one, stated where used).
 *   - The pages only name the format "MXFP4"; the bit-level meaning of an
 *     E2M1 element, an E8M0 scale, an E4M3 element and the scalar-to-MX
 *     conversion rule are those of the OCP Microscaling Formats (MX)
 *     Specification v1.0, which that name refers to.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Elements per MX block (one E8M0 scale per block). */
#define ORC_MX_BLOCK 32

/* ---- element and scale codecs (OCP MX v1.0 element/scale formats) ---- */
double orc_e2m1_value(uint32_t nibble);      /* 4-bit code -> value          */
double orc_e8m0_value(uint32_t byte);        /* 2^(byte-127); NaN for 0xFF    */
double orc_e4m3_value(uint32_t byte);        /* OCP E4M3 (no inf); NaN 0x7F/0xFF */

/* Nearest-even rounding of one already-scaled value onto the element grid.
 * Returns the code (sign in bit 3 for E2M1, bit 7 for E4M3).  Saturates. */
uint32_t orc_e2m1_round(double q);
uint32_t orc_e4m3_round(double q);

/* Row-major MXFP4 tensor [rows][K]: packed [rows][K/2] (element kk in byte
 * kk/2, low nibble for even kk), scales [rows][K/32]. */
void orc_dequant_mxfp4(const uint8_t* packed, const uint8_t* scales,
                       int64_t rows, int64_t K, double* out);
void orc_quant_mxfp4(const float* w, int64_t rows, int64_t K,
                     uint8_t* packed, uint8_t* scales);

/* Row-major MXFP8 (E4M3) tensor [rows][K]: codes [rows][K], scales [rows][K/32]. */
void orc_quant_mxfp8(const double* v, int64_t rows, int64_t K,
                     uint8_t* codes, uint8_t* scales);
void orc_dequant_mxfp8(const uint8_t* codes, const uint8_t* scales,
                       int64_t rows, int64_t K, double* out);

/* ---- router projection (in front of the routing) ---- */
/* logits[T][E] = x[T][d] . W[E][d]^T in double from bf16 bit patterns; the
 * optional absdot[T][E] (NULL to skip) gets sum_i |x[t][i] * W[e][i]|, the
 * scale of any rounding error in a lower-precision evaluation. */
void orc_router_logits(const uint16_t* x_bf16, const uint16_t* w_bf16, int32_t T, int32_t d,
                       int32_t E, double* logits, double* absdot);

/* ---- DFlash verify acceptance (rejection sampling over a block) ---- */
/* B sequences, blocks of G draft tokens, vocabulary V.  draft [B][G],
 * p_draft [B][G][V], p_target [B][G+1][V], u [B][G], r [B] (uniforms in
 * [0, 1)).  Out: n_accepted [B] (0..G) and next_token [B] (-1 if the row
 * drawn from has no positive entry).  Readings for inputs outside the
 * method's domain: a draft token outside [0, V) is rejected; entries that
 * are not positive (NaN included) weigh nothing; r is clamped into [0, 1). */
void orc_dflash_accept(int32_t B, int32_t G, int32_t V, const int32_t* draft, const float* p_draft,
                       const float* p_target, const float* u, const float* r, int32_t* n_accepted,
                       int32_t* next_token);

/* ---- routing and permutation ---- */
void orc_route(const float* logits, int32_t T, int32_t E, int32_t k,
               int32_t* topk_ids, double* topk_w);
void orc_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                 int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                 int32_t* inverse);

/* ---- whole expert layer ---- */
enum { ORC_ACT_BF16 = 0, ORC_ACT_MXFP8 = 1 };

/* y[T][d] (double).  Weights: gate/up packed [E][f][d/2] + scales [E][f][d/32],
 * down packed [E][d][f/2] + scales [E][d][f/32].  x is bf16 bit patterns.
 * Optional outputs (NULL to skip): topk ids/weights [T][k], h [T][k][f]
 * (after the optional MXFP8 round trip).  nthreads <= 0: OpenMP default.
 * Returns the number of OpenMP threads used, or -1 on a bad argument. */
int32_t orc_moe_forward(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k,
                        int32_t act_mode, const uint16_t* x_bf16,
                        const float* logits,
                        const uint8_t* w_gate, const uint8_t* w_gate_scale,
                        const uint8_t* w_up, const uint8_t* w_up_scale,
                        const uint8_t* w_down, const uint8_t* w_down_scale,
                        double* y, int32_t* topk_ids, double* topk_w,
                        double* h, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
