/*
 * sparse_moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts
 * feed-forward layer with ggml Q4_0 experts (Gemma 4 26B-A4B shape).
 *
 * The layer, as the model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP
 * assistant and vision, NInfer v3 artifact" describes it (intro and table
 * "What is inside"): 128 routed experts per block, stored expert-major in
 * ggml Q4_0 blocks that are multiplied in place (never requantised), each
 * expert a [gate; up] parent of 2 x 704 rows and a down matrix of 2,816 rows;
 * router, router scale and expert scales in FP32.  "Gemma 4 26B A4B lands on
 * Hugging Face ...", section "How it works": about 4B of 26B parameters are
 * active per token.
 *
 * Four calls make one layer, in this order:
 *   moe_router_topk      logits = x W_r^T (FP32), top-K experts, softmax weights
 *   moe_permute          stable counting sort of the T*K (token, k) slots by expert
 *   moe_expert_ffn_q4_0  per slot: h = GELU_tanh(x Wg^T) * (x Wu^T), y = h Wd^T
 *   moe_combine          out[t] = sum_k w[t,k] * scale[e] * y[slot]
 * moe_route does the first two in one call (one kernel for up to 8 tokens).
 * Also: moe_rmsnorm, the pre-norm of a stack of such layers, and
 * moe_linear_q4_0, a plain Q4_0 linear layer on the same kernels (a block's
 * Q, K, V parent).
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers owned by the caller (unless a parameter says
 *    host).  The library never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on it and returns; device faults surface at the
 *    caller's next synchronisation.
 *  - Arguments are validated before anything is enqueued; on error nothing is
 *    enqueued and the status says why.  A launch failure returns MOE_ERR_HIP.
 *  - T == 0 is a valid no-op (returns MOE_OK, touches nothing).
 *  - Shapes: 1 <= K <= E <= MOE_MAX_E, K <= MOE_MAX_K, H % 32 == 0,
 *    I % 32 == 0, H <= MOE_MAX_H, I <= MOE_MAX_I, T*K < 2^31.
 *  - Every device pointer must be 16-byte aligned.
 *  - Activations: MOE_F32 (float) or MOE_BF16 (bfloat16 bits in uint16).
 *  - Calls are thread-safe; calls that share a workspace must be ordered on
 *    one stream.
 *  - Results are deterministic: the same inputs give bitwise the same outputs.
 *  - Below 64 tokens a token's logits, top-K and outputs do not depend on the
 *    other tokens of the batch (bitwise), so a verification batch reproduces
 *    the single-token decode (model card, sections "Speculative decoding" and
 *    "Quality").
 */
#ifndef SPARSE_MOE_H
#define SPARSE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1
#define MOE_MAX_E 256
#define MOE_MAX_K 16
#define MOE_MAX_H 4096
#define MOE_MAX_I 4096
#define MOE_MAX_LINEAR_ROWS 65536
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20) /* static workspace per GPU, see below */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    MOE_ERR_UNSUPPORTED = 4, /* unknown dtype or option */
    MOE_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    MOE_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    MOE_ERR_SCRATCH = 7      /* needs more than the no-allocation entry point's scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Static string describing a status code (never NULL). */
const char* moe_status_string(int status);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/*
 * Router and top-K (model card table "What is inside": FP32 router and router
 * scale; the layer routes each token to its top-K experts with softmax weights
 * renormalised over the K chosen, the plainest reading of a top-k softmax
 * router with the per-expert scale applied later, in moe_combine).
 *
 *   x          [T, H] activations of type x_dt (read only when W_r != NULL)
 *   W_r        [E, H] fp32 router weight, row-major; NULL selects the bypass
 *              mode in which `logits` is an INPUT holding [T, E] fp32 logits
 *   r_scale    [H] fp32 per-channel multiplier of the router input, or NULL (= 1)
 *   logit_bias [E] fp32 added to every token's logits, or NULL (= 0)
 *   logits     [T, E] fp32: OUTPUT x (r_scale * W_r)^T + bias when W_r != NULL,
 *              INPUT otherwise.  Required.
 *   topk_ids   [T, K] int32 OUTPUT: experts by descending logit, equal logits
 *              in ascending expert order
 *   topk_w     [T, K] fp32 OUTPUT: w[t,k] = exp(l_k - l_0) / sum_j exp(l_j - l_0)
 *              over the K selected logits (sums to 1 per token)
 * Logits are accumulated in fp32.  NaN logits give undefined ids.
 */
moe_status moe_router_topk(const void* x, int x_dt, int64_t T, int32_t H, const float* W_r,
                           const float* r_scale, const float* logit_bias, int32_t E, int32_t K,
                           float* logits, int32_t* topk_ids, float* topk_w, void* stream);

/*
 * Token -> expert permutation: a stable counting sort of the N = T*K slots
 * s = t*K + k by expert topk_ids[s] (ids must lie in [0, E)).
 *
 *   expert_offsets [E+1] int32 OUTPUT: exclusive prefix sum of per-expert slot
 *                  counts; expert_offsets[E] == N
 *   sorted_slots   [N] int32 OUTPUT: the slot stored at sorted position p;
 *                  within one expert, slots ascend
 *   slot_pos       [N] int32 OUTPUT: inverse map, sorted position of slot s
 *   ws, ws_bytes   device workspace of at least
 *                  moe_permute_workspace_bytes(T, K, E) bytes (may be NULL
 *                  when that is 0); contents need no initialisation
 * Results are unique (bit-exact, no tie ambiguity).
 */
size_t moe_permute_workspace_bytes(int64_t T, int32_t K, int32_t E);
moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E,
                       int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_pos,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Routing in one call: moe_router_topk followed by moe_permute, with the same
 * results (same arguments as those two calls; W_r == NULL again selects
 * injected logits).  For T <= 8 and a router weight, one kernel does all of it:
 * every workgroup computes a share of the router logits and the last one to
 * finish (counted by an atomic in the workspace) runs top-K and the
 * permutation.  This is the decode path; it saves two kernel boundaries.
 *
 *   ws   device workspace of at least moe_route_workspace_bytes(T, K, E) bytes,
 *        ZERO-FILLED before its first use; every call leaves it zero-filled
 *        again.  Calls sharing a workspace must be ordered on one stream.
 */
size_t moe_route_workspace_bytes(int64_t T, int32_t K, int32_t E);
moe_status moe_route(const void* x, int x_dt, int64_t T, int32_t H, const float* W_r,
                     const float* r_scale, const float* logit_bias, int32_t E, int32_t K,
                     float* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                     int32_t* sorted_slots, int32_t* slot_pos, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * Expert FFN on Q4_0 weights read in place (model card intro: the release's
 * ggml blocks are kept byte for byte and multiplied in place; table "What is
 * inside": expert-major [gate; up] 2 x I rows and down H rows).
 *
 *   x          [T, H] activations of type x_dt
 *   w_gate_up  raw Q4_0 bytes [E][2I rows][H/32 blocks][18]: rows 0..I-1 gate,
 *              rows I..2I-1 up.  Block = fp16 scale d (little-endian) + 16 bytes
 *              qs; element j = (qs[j] & 15) - 8, element j+16 = (qs[j] >> 4) - 8,
 *              times d.
 *   w_down     raw Q4_0 bytes [E][H rows][I/32 blocks][18]
 *   expert_offsets, sorted_slots   as produced by moe_permute
 *   y_sorted   [N, H] fp32 OUTPUT: row p = expert output of slot sorted_slots[p]
 *              for the expert that owns position p
 *   ws         device workspace of at least
 *              moe_expert_ffn_q4_0_workspace_bytes(T, K, H, I, E, x_dt) bytes
 *              (holds the hidden h); contents need no initialisation
 * Per slot: g = Wg x, u = Wu x, h = GELU_tanh(g) * u rounded to x_dt (the
 * hidden is materialised in the activation type), y = Wd h; GELU_tanh(z) =
 * z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).  Dequantised weights are never
 * rounded; accumulation is fp32.  The two paths treat the activations
 * differently:
 *  - GEMV path (fewer than 64 tokens, or fp32 activations, or H or I not a
 *    multiple of 64): each 32-element block of the activations (x for
 *    gate/up, h for down) is first rounded to 15-bit fixed point relative to
 *    the block's largest magnitude m, n = rint(v * 30583 / m), an error of at
 *    most m / 61166 per element; the block's products with the 4-bit codes
 *    are then exact integers, scaled by d * m / 30583 in fp32.
 *  - MFMA path (bf16 activations, at least 64 tokens, H and I multiples of
 *    64): the bf16 activations enter bf16 MFMAs exactly (exact products, fp32
 *    accumulation per Q4_0 block, then times d).
 */
size_t moe_expert_ffn_q4_0_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t I,
                                           int32_t E, int x_dt);
moe_status moe_expert_ffn_q4_0(const void* x, int x_dt, int64_t T, int32_t H,
                               const void* w_gate_up, const void* w_down, int32_t I, int32_t E,
                               int32_t K, const int32_t* expert_offsets,
                               const int32_t* sorted_slots, float* y_sorted, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * One whole decode layer in one call: the results of moe_route,
 * moe_expert_ffn_q4_0 and moe_combine, bit for bit, for decode and
 * verification batches (model card intro: one to eight concurrent requests;
 * sections "Speed" and "Speculative decoding": decode speed, and drafts of a
 * few tokens verified in one pass).  Three kernels instead of five: the router
 * logits; gate/up with top-K and the permutation computed inside every
 * workgroup (no hand-off through a completion counter); down with the
 * weighted combine inside (each workgroup owns a few output rows of one token
 * and sums its K experts there, so no per-slot output y is stored).  One
 * token at 2048 < H <= 4096, 512 < I <= 1024 and K <= 8 (the Gemma shape)
 * runs gate/up and down in ONE launch: the down workgroups fetch their
 * weights, then wait on completion counters bumped by the gate/up workgroups
 * (a bounded wait; see ws below).
 *
 *   Arguments are those of the three calls: W_r == NULL selects injected
 *   logits (then `logits` is an INPUT); logits, topk_ids, topk_w,
 *   expert_offsets, sorted_slots and slot_pos are OUTPUTS as there (required);
 *   out_f32 / out_act / residual as in moe_combine (at least one output).
 *   ws   >= moe_layer_decode_workspace_bytes(T, K, H, I, E, x_dt) bytes,
 *        16-byte aligned: a 16 KiB header of completion counters (zeroed by
 *        the call itself), then the hidden h; contents need no
 *        initialisation.  After the call, int 1 of ws is non-zero only if the
 *        one-launch path's bounded wait expired (then the output is not
 *        written); it never does while the launch runs alone on the GPU's
 *        queue, since every waiting workgroup was dispatched after the
 *        workgroups it waits for.
 * Supported shapes: 1 <= T <= 8, T * K <= 64, H and I multiples of 64, and
 * K * (I / 32) * 68 bytes of staged hidden digits <= 64 KiB; other shapes
 * return MOE_ERR_UNSUPPORTED (use the separate calls).  The hidden h goes
 * through the decode GEMV's 15-bit block fixed point, as in
 * moe_expert_ffn_q4_0's GEMV path.
 */
size_t moe_layer_decode_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t I, int32_t E,
                                        int x_dt);
moe_status moe_layer_decode(const void* x, int x_dt, int64_t T, int32_t H, const float* W_r,
                            const float* r_scale, const float* logit_bias, int32_t E, int32_t K,
                            const void* w_gate_up, const void* w_down, int32_t I,
                            const float* expert_scale, float* logits, int32_t* topk_ids,
                            float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                            int32_t* slot_pos, const void* residual, int residual_dt,
                            float* out_f32, void* out_act, int out_dt, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * moe_expert_ffn_q4_0 without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * moe_expert_ffn_q4_0 (bitwise), with the workspace taken from a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds once per
 * GPU until the process ends.  Nothing is allocated: the array's address is
 * looked up once per device (hipGetSymbolAddress) and kept.
 *  - Returns MOE_ERR_SCRATCH, enqueueing nothing, when
 *    moe_expert_ffn_q4_0_workspace_bytes(T, K, H, I, E, x_dt) exceeds the
 *    array (at the Gemma shape: about 927 tokens on the bf16 MFMA path; every
 *    decode batch of fewer than 64 tokens fits).
 *  - Every call on one GPU shares that GPU's array, and the array keeps the
 *    last call's contents (the workspace needs no initialisation).  Calls
 *    whose execution overlaps on one GPU (other streams, other threads) race
 *    on it: order them on one stream.
 */
moe_status moe_expert_ffn_q4_0_noalloc(const void* x, int x_dt, int64_t T, int32_t H,
                                       const void* w_gate_up, const void* w_down, int32_t I,
                                       int32_t E, int32_t K, const int32_t* expert_offsets,
                                       const int32_t* sorted_slots, float* y_sorted,
                                       void* stream);

/*
 * Plain Q4_0 linear layer (model card table "What is inside": the Q, K and V
 * rows of a block form one Q4_0 parent, stored and multiplied like the
 * experts' matrices).
 *
 *   x   [T, H] of type x_dt (fp32 or bf16), H % 32 == 0, H <= MOE_MAX_I
 *   W   raw Q4_0 bytes [R rows][H/32 blocks][18], read in place;
 *       1 <= R <= MOE_MAX_LINEAR_ROWS
 *   y   [T, R] fp32 OUTPUT: y[t, r] = sum_j W[r, j] x[t, j]
 *   ws  >= moe_linear_q4_0_workspace_bytes(T, H, R, x_dt) bytes, 16-byte
 *       aligned; contents need no initialisation
 * The same kernels as the experts' down product (one expert holding every
 * token): for few tokens the Q4_0 GEMV, which rounds each 32-element block of x
 * to 15-bit fixed point relative to its largest magnitude m (error <= m / 61166
 * per element) and then takes exact integer block products; for bf16
 * activations from 64 tokens (H % 64 == 0 and R % 16 == 0) exact bf16 MFMA
 * products.  fp32 accumulation, weights never rounded.
 */
size_t moe_linear_q4_0_workspace_bytes(int64_t T, int32_t H, int32_t R, int x_dt);
moe_status moe_linear_q4_0(const void* x, int x_dt, int64_t T, int32_t H, const void* W,
                           int32_t R, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Weighted combine (model card table "What is inside": FP32 expert scales).
 *
 *   out[t, o] = sum_{k=0..K-1} (topk_w[t,k] * expert_scale[topk_ids[t,k]])
 *                              * y_sorted[slot_pos[t*K+k], o]       (fixed k order)
 *   expert_scale  [E] fp32 or NULL (= 1)
 *   residual      [T, H] of type residual_dt, or NULL
 *   out_f32       [T, H] fp32 OUTPUT of the sum above (never includes the
 *                 residual), or NULL
 *   out_act       [T, H] OUTPUT of type out_dt: (residual + out) rounded to
 *                 nearest even, or NULL.  At least one output is required.
 */
moe_status moe_combine(const float* y_sorted, const int32_t* slot_pos, const int32_t* topk_ids,
                       const float* topk_w, const float* expert_scale, int64_t T, int32_t K,
                       int32_t H, const void* residual, int residual_dt, float* out_f32,
                       void* out_act, int out_dt, void* stream);

/*
 * RMSNorm before a layer of a stack (model card table "What is inside": FP32
 * norms): out[t,:] = x[t,:] * (mean_j x[t,j]^2 + eps)^-1/2 * w, computed in
 * fp32 and rounded to out_dt.  w [H] fp32.
 */
moe_status moe_rmsnorm(const void* x, int x_dt, const float* w, float eps, int64_t T, int32_t H,
                       void* out, int out_dt, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_MOE_H */
