/*
 * moe_oracle.h -- plain, slow, single-threaded CPU reference of the routed
 * Mixture-of-Experts feed-forward layer of Gemma 4 26B-A4B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library (no headers, no helpers, no tables).
 *
 * Sources of each step (page titles as published):
 *  - "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision, NInfer v3
 *    artifact", intro: every matrix keeps the release's ggml blocks byte for
 *    byte and the engine multiplies the blocks in place (no requantisation);
 *    table "What is inside": 128 routed experts per block, Q4_0,
 *    expert-major, a [gate; up] parent of 2 x 704 rows and a down matrix of
 *    2,816 rows; norms, router, router scale and expert scales are FP32.
 *  - "Gemma 4 26B A4B lands on Hugging Face ...", section "How it works":
 *    a Mixture-of-Experts model, about 4B of 26B parameters active per token.
 *  Steps the pages leave open are taken from the layer's workload definition
 *  and are listed as readings where they are used (top-k renormalised
 *  softmax, GELU-tanh(gate) * up, expert scale in the combine, RMSNorm).
 *
 * All arithmetic is IEEE binary64; inputs are decoded exactly; results that
 * the layer materialises in a narrower type (the hidden h, the stack's
 * residual stream) are rounded to that type round-to-nearest-even.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* ---- number formats ---------------------------------------------------- */
double   orc_f16_to_f64(uint16_t h);          /* IEEE binary16, subnormals included */
double   orc_bf16_to_f64(uint16_t b);         /* upper half of a binary32 */
uint16_t orc_f64_to_bf16(double v);           /* round to nearest, ties to even */
double   orc_round_act(double v, int act);    /* v rounded to fp32 or bf16, as double */
double   orc_load_act(const void* base, int act, int64_t idx);

/* ---- Q4_0 --------------------------------------------------------------- */
/* One 18-byte ggml Q4_0 block: little-endian fp16 scale d, then 16 bytes qs.
 * Element j (0..15) is the low nibble of qs[j], element j+16 the high nibble;
 * value = (nibble - 8) * d. */
void     orc_q4_0_decode(const uint8_t* blk, double out[32]);

/* GELU with the tanh approximation: 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3))). */
double   orc_gelu_tanh(double z);

/* ---- steps of the layer -------------------------------------------------- */
/* logits[t,e] = sum_j x[t,j] * r_scale[j] * W_r[e,j] + bias[e]; r_scale, bias nullable. */
int orc_router_logits(const void* x, int x_dt, int64_t T, int H, const float* w_r,
                      const float* r_scale, const float* bias, int E, double* logits);

/* ids[t,:] = first K of a stable descending sort of logits[t,:] (equal logits:
 * lower expert first); p = softmax over all E; w[t,k] = p[ids[t,k]] / sum_k p[ids[t,k]]. */
int orc_topk_softmax(const double* logits, int64_t T, int E, int K, int32_t* ids, double* w);

/* The weights alone, for given expert ids (the second half of orc_topk_softmax). */
int orc_topk_weights(const double* logits, int64_t T, int E, int K, const int32_t* ids, double* w);

/* Stable counting sort of slots s = t*K + k by ids[s]: offsets[E+1] exclusive
 * prefix of per-expert counts, sorted_slots[p] = slot at position p,
 * slot_pos[s] = position of slot s. */
int orc_permute(const int32_t* ids, int64_t T, int K, int E, int32_t* offsets,
                int32_t* sorted_slots, int32_t* slot_pos);

/* One token through expert e: g = Wg x, u = Wu x (rows 0..I-1 and I..2I-1 of
 * the [gate; up] parent), h = act_round(gelu_tanh(g) * u), y = Wd h.
 * x_row points at H activations of type x_dt; h_out (I) and y_out (H) nullable. */
int orc_expert_ffn_token(const void* x_row, int x_dt, int H, const uint8_t* w_gate_up,
                         const uint8_t* w_down, int I, int e, double* h_out, double* y_out);

/* Q4_0 linear layer: y[t,r] = sum_j W[r,j] x[t,j] for r < R, W a matrix of R
 * rows of H/32 Q4_0 blocks used in place (model card, table "What is inside":
 * the Q, K and V rows of a block are one Q4_0 parent, like the experts'), fp64
 * accumulation; y is [T, R]. */
int orc_linear_q4_0(const void* x, int x_dt, int64_t T, int H, const uint8_t* w, int R, double* y);

/* y_sorted[p,:] = expert output for slot sorted_slots[p] (expert owning position p).
 * slot_mask (nullable, indexed by slot) restricts the work to selected slots;
 * rows of unselected slots are left untouched. */
int orc_expert_ffn(const void* x, int x_dt, int64_t T, int H, const uint8_t* w_gate_up,
                   const uint8_t* w_down, int I, int E, int K, const int32_t* offsets,
                   const int32_t* sorted_slots, const uint8_t* slot_mask, double* y_sorted);

/* out[t,o] = sum_{k=0..K-1} (w[t,k] * scale[ids[t,k]]) * y_sorted[slot_pos[t*K+k], o];
 * scale nullable (= 1); token_mask nullable (rows of unselected tokens untouched). */
int orc_combine(const double* y_sorted, const int32_t* slot_pos, const int32_t* ids,
                const double* w, const float* scale, int64_t T, int K, int H,
                const uint8_t* token_mask, double* out);

/* out[t,:] = bf16( x[t,:] * (mean_j x[t,j]^2 + eps)^-1/2 * w ). */
int orc_rmsnorm(const void* x, int x_dt, const float* w, double eps, int64_t T, int H,
                uint16_t* out_bf16);

/* Whole layer.  w_r NULL: logits_in [T,E] fp32 are the router logits.
 * token_mask (nullable) restricts the expert FFN and combine to selected tokens
 * (routing and the permutation always cover every token).
 * Outputs: logits (nullable, [T,E]), ids [T,K], w [T,K], offsets [E+1],
 * sorted_slots [T*K], slot_pos [T*K], out [T,H] (only selected rows written). */
int orc_moe_layer(const void* x, int x_dt, int64_t T, int H, const float* w_r,
                  const float* logits_in, const float* r_scale, const float* bias, int E, int K,
                  const uint8_t* w_gate_up, const uint8_t* w_down, int I, const float* scale,
                  const uint8_t* token_mask, double* logits, int32_t* ids, double* w,
                  int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, double* out);

/* Residual add between the blocks of the stack: x_next = bf16(x + out), with
 * x the bf16 residual stream and out the layer's combined output (binary64),
 * added exactly and rounded once, to nearest even.  token_mask nullable (rows
 * of unselected tokens untouched). */
int orc_residual(const uint16_t* x_bf16, const double* out, int64_t T, int H,
                 const uint8_t* token_mask, uint16_t* x_next);

/* One block of the stack, pre-norm: xhat = RMSNorm(x) (bf16), the routed
 * layer on xhat (router with the additive prior `bias`, experts and the
 * combine as in orc_moe_layer), then x_next = bf16(x + out).  token_mask as in
 * orc_moe_layer (routing covers every token; the FFN, the combine and the
 * residual only the selected ones).  xhat_out, ids, out: nullable [T,H] bf16,
 * [T,K] int32, [T,H] binary64 copies of the intermediate results. */
int orc_stack_layer(const uint16_t* x_bf16, int64_t T, int H, const float* rms_w, double eps,
                    const float* w_r, const float* bias, int E, int K, const uint8_t* w_gate_up,
                    const uint8_t* w_down, int I, const float* scale, const uint8_t* token_mask,
                    uint16_t* xhat_out, int32_t* ids_out, double* out_out, uint16_t* x_next);

#ifdef __cplusplus
}
#endif
#endif
