// C ABI of the routed-MoE library: argument validation, workspace layout and
// dispatch to the gfx950 kernels.  Nothing here allocates, frees or
// synchronises; every call only enqueues on the caller's stream.
#include <algorithm>
#include <mutex>

#include "kernels.h"

// Workspace of moe_expert_ffn_q4_0_noalloc: one copy per GPU, held until the
// process ends.  In host code `scratch` only names the symbol; its device
// address on each GPU comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_ekh(int64_t T, int32_t K, int32_t E) {
    if (T < 0 || T > (int64_t)0x7FFFFFFF) return MOE_ERR_SHAPE;
    if (E < 1 || E > MOE_MAX_E || K < 1 || K > E || K > MOE_MAX_K) return MOE_ERR_SHAPE;
    if (T * (int64_t)K > (int64_t)0x7FFFFFFF) return MOE_ERR_SHAPE;
    return MOE_OK;
}

moe_status check_dim(int32_t D, int32_t maxD) {
    return (D < 32 || D % 32 != 0 || D > maxD) ? MOE_ERR_SHAPE : MOE_OK;
}

// Device address of `scratch` on the device that owns `stream` (the current
// device for the null stream), looked up once per device with that device
// current and kept.
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[SCRATCH_MAX_DEVICES];

moe_status scratch_address(hipStream_t stream, void** out) {
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
    dev = cur;
    if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
        if (e != hipSuccess || !p) return MOE_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of range or inconsistent";
        case MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
        case MOE_ERR_UNSUPPORTED: return "unsupported dtype or option";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "the HIP runtime reported a launch error";
        case MOE_ERR_SCRATCH:
            return "the call needs more workspace than the static scratch of the "
                   "no-allocation entry point holds (MOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_router_topk(const void* x, int x_dt, int64_t T, int32_t H, const float* W_r,
                           const float* r_scale, const float* logit_bias, int32_t E, int32_t K,
                           float* logits, int32_t* topk_ids, float* topk_w, void* stream) {
    moe_status s = check_ekh(T, K, E);
    if (s != MOE_OK) return s;
    if (W_r && (s = check_dim(H, MOE_MAX_H)) != MOE_OK) return s;
    if (!dtype_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w || (W_r && !x)) return MOE_ERR_NULL;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_ERR_ALIGN;
    if (W_r && (!aligned16(x) || !aligned16(W_r) || (r_scale && !aligned16(r_scale)) ||
                (logit_bias && !aligned16(logit_bias))))
        return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    if (W_r) {
        s = hip_status(moe::launch_router_logits(x, x_dt, T, H, W_r, r_scale, logit_bias, E, logits, st));
        if (s != MOE_OK) return s;
    }
    return hip_status(moe::launch_topk(logits, T, E, K, topk_ids, topk_w, st));
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t K, int32_t E) {
    if (check_ekh(T, K, E) != MOE_OK) return 0;
    return round_up(moe::permute_ws_bytes(T * K, E), 256);
}

moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E,
                       int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_pos, void* ws,
                       size_t ws_bytes, void* stream) {
    moe_status s = check_ekh(T, K, E);
    if (s != MOE_OK) return s;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !expert_offsets || !sorted_slots || !slot_pos) return MOE_ERR_NULL;
    if (!aligned16(topk_ids) || !aligned16(expert_offsets) || !aligned16(sorted_slots) ||
        !aligned16(slot_pos))
        return MOE_ERR_ALIGN;
    const size_t need = moe_permute_workspace_bytes(T, K, E);
    if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    if (ws && !aligned16(ws)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_permute(topk_ids, (int)(T * K), E, expert_offsets, sorted_slots,
                                          slot_pos, ws, (hipStream_t)stream));
}

size_t moe_route_workspace_bytes(int64_t T, int32_t K, int32_t E) {
    if (check_ekh(T, K, E) != MOE_OK) return 0;
    // [0, 256): completion counter of the fused few-token kernel; then the
    // workspace of the multi-tile permutation
    return 256 + round_up(moe::permute_ws_bytes(T * K, E), 256);
}

moe_status moe_route(const void* x, int x_dt, int64_t T, int32_t H, const float* W_r,
                     const float* r_scale, const float* logit_bias, int32_t E, int32_t K,
                     float* logits, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                     int32_t* sorted_slots, int32_t* slot_pos, void* ws, size_t ws_bytes,
                     void* stream) {
    moe_status s = check_ekh(T, K, E);
    if (s != MOE_OK) return s;
    if (W_r && (s = check_dim(H, MOE_MAX_H)) != MOE_OK) return s;
    if (!dtype_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w || (W_r && !x) || !expert_offsets || !sorted_slots ||
        !slot_pos)
        return MOE_ERR_NULL;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) ||
        !aligned16(expert_offsets) || !aligned16(sorted_slots) || !aligned16(slot_pos))
        return MOE_ERR_ALIGN;
    if (W_r && (!aligned16(x) || !aligned16(W_r) || (r_scale && !aligned16(r_scale)) ||
                (logit_bias && !aligned16(logit_bias))))
        return MOE_ERR_ALIGN;
    const size_t need = moe_route_workspace_bytes(T, K, E);
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    const int N = (int)(T * K);
    if (W_r && T <= moe::ROUTER_GEMV_MAX_T && N <= moe::PERM_TILE)
        return hip_status(moe::launch_route_small(x, x_dt, (int)T, H, W_r, r_scale, logit_bias, E, K,
                                                  logits, topk_ids, topk_w, expert_offsets,
                                                  sorted_slots, slot_pos, (int*)ws, st));
    if (W_r && (s = hip_status(moe::launch_router_logits(x, x_dt, T, H, W_r, r_scale, logit_bias, E,
                                                        logits, st))) != MOE_OK)
        return s;
    if ((s = hip_status(moe::launch_topk(logits, T, E, K, topk_ids, topk_w, st))) != MOE_OK) return s;
    return hip_status(moe::launch_permute(topk_ids, N, E, expert_offsets, sorted_slots, slot_pos,
                                          (uint8_t*)ws + 256, st));
}

size_t moe_expert_ffn_q4_0_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t I, int32_t E,
                                           int x_dt) {
    if (check_ekh(T, K, E) != MOE_OK || check_dim(H, MOE_MAX_H) != MOE_OK ||
        check_dim(I, MOE_MAX_I) != MOE_OK || !dtype_ok(x_dt))
        return 0;
    // GEMV path: hidden h [T*K, I] in the activation dtype.  MFMA path (bf16
    // activations, many tokens): activations and hidden in the MFMA block
    // order with their block sums.
    const size_t gemv = round_up((size_t)(T * K) * (size_t)I * (x_dt == MOE_F32 ? 4 : 2), 256);
    if (moe::ffn_use_mfma(x_dt, T, H, I))
        return std::max(gemv, moe::ffn_mfma_ws_bytes(T, H, I, T * K));
    return gemv;
}

moe_status moe_expert_ffn_q4_0(const void* x, int x_dt, int64_t T, int32_t H,
                               const void* w_gate_up, const void* w_down, int32_t I, int32_t E,
                               int32_t K, const int32_t* expert_offsets,
                               const int32_t* sorted_slots, float* y_sorted, void* ws,
                               size_t ws_bytes, void* stream) {
    moe_status s = check_ekh(T, K, E);
    if (s != MOE_OK) return s;
    if ((s = check_dim(H, MOE_MAX_H)) != MOE_OK || (s = check_dim(I, MOE_MAX_I)) != MOE_OK) return s;
    if (!dtype_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !w_gate_up || !w_down || !expert_offsets || !sorted_slots || !y_sorted)
        return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) ||
        !aligned16(expert_offsets) || !aligned16(sorted_slots) || !aligned16(y_sorted))
        return MOE_ERR_ALIGN;
    const size_t need = moe_expert_ffn_q4_0_workspace_bytes(T, K, H, I, E, x_dt);
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    if (moe::ffn_use_mfma(x_dt, T, H, I))
        return hip_status(moe::launch_ffn_mfma(x, T, H, (const uint8_t*)w_gate_up,
                                               (const uint8_t*)w_down, I, E, K, (int)(T * K),
                                               expert_offsets, sorted_slots, ws, y_sorted,
                                               (hipStream_t)stream));
    return hip_status(moe::launch_ffn_gemv(x, x_dt, T, H, (const uint8_t*)w_gate_up,
                                           (const uint8_t*)w_down, I, E, K, (int)(T * K),
                                           expert_offsets, sorted_slots, ws, y_sorted,
                                           (hipStream_t)stream));
}

size_t moe_layer_decode_workspace_bytes(int64_t T, int32_t K, int32_t H, int32_t I, int32_t E,
                                        int x_dt) {
    if (check_ekh(T, K, E) != MOE_OK || check_dim(H, MOE_MAX_H) != MOE_OK ||
        check_dim(I, MOE_MAX_I) != MOE_OK || !dtype_ok(x_dt))
        return 0;
    // [0, DECODE_CTR_BYTES): the one-token path's completion counters and
    // timeout flag; then the hidden h [T*K, I] in the activation dtype, in
    // sorted-slot order
    return moe::DECODE_CTR_BYTES + round_up((size_t)(T * K) * (size_t)I * (x_dt == MOE_F32 ? 4 : 2), 256);
}

moe_status moe_layer_decode(const void* x, int x_dt, int64_t T, int32_t H, const float* W_r,
                            const float* r_scale, const float* logit_bias, int32_t E, int32_t K,
                            const void* w_gate_up, const void* w_down, int32_t I,
                            const float* expert_scale, float* logits, int32_t* topk_ids,
                            float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                            int32_t* slot_pos, const void* residual, int residual_dt,
                            float* out_f32, void* out_act, int out_dt, void* ws, size_t ws_bytes,
                            void* stream) {
    moe_status s = check_ekh(T, K, E);
    if (s != MOE_OK) return s;
    if ((s = check_dim(H, MOE_MAX_H)) != MOE_OK || (s = check_dim(I, MOE_MAX_I)) != MOE_OK) return s;
    if (!dtype_ok(x_dt) || !dtype_ok(out_dt) || (residual && !dtype_ok(residual_dt)))
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!moe::decode_layer_supported(T, H, I, K)) return MOE_ERR_UNSUPPORTED;
    if (!x || !logits || !topk_ids || !topk_w || !expert_offsets || !sorted_slots || !slot_pos ||
        !w_gate_up || !w_down || (!out_f32 && !out_act))
        return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w) ||
        !aligned16(expert_offsets) || !aligned16(sorted_slots) || !aligned16(slot_pos) ||
        !aligned16(w_gate_up) || !aligned16(w_down) ||
        (W_r && (!aligned16(W_r) || (r_scale && !aligned16(r_scale)) ||
                 (logit_bias && !aligned16(logit_bias)))) ||
        (expert_scale && !aligned16(expert_scale)) || (residual && !aligned16(residual)) ||
        (out_f32 && !aligned16(out_f32)) || (out_act && !aligned16(out_act)))
        return MOE_ERR_ALIGN;
    const size_t need = moe_layer_decode_workspace_bytes(T, K, H, I, E, x_dt);
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    int* ctr = (int*)ws;  // zeroed by this call's router launch (or a launch of its own)
    if (W_r) {
        if ((s = hip_status(moe::launch_router_logits(x, x_dt, T, H, W_r, r_scale, logit_bias, E,
                                                      logits, st, ctr))) != MOE_OK)
            return s;
    } else if ((s = hip_status(moe::launch_zero_decode_ctr(ctr, st))) != MOE_OK) {
        return s;
    }
    return hip_status(moe::launch_decode_layer(
        x, x_dt, (int)T, H, logits, E, K, (const uint8_t*)w_gate_up, (const uint8_t*)w_down, I,
        expert_scale, topk_ids, topk_w, expert_offsets, sorted_slots, slot_pos, residual,
        residual_dt, out_f32, out_act, out_dt, (uint8_t*)ws + moe::DECODE_CTR_BYTES, ctr, st));
}

moe_status moe_expert_ffn_q4_0_noalloc(const void* x, int x_dt, int64_t T, int32_t H,
                                       const void* w_gate_up, const void* w_down, int32_t I,
                                       int32_t E, int32_t K, const int32_t* expert_offsets,
                                       const int32_t* sorted_slots, float* y_sorted,
                                       void* stream) {
    moe_status s = check_ekh(T, K, E);
    if (s != MOE_OK) return s;
    if ((s = check_dim(H, MOE_MAX_H)) != MOE_OK || (s = check_dim(I, MOE_MAX_I)) != MOE_OK) return s;
    if (!dtype_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (moe_expert_ffn_q4_0_workspace_bytes(T, K, H, I, E, x_dt) > MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_SCRATCH;
    if (!x || !w_gate_up || !w_down || !expert_offsets || !sorted_slots || !y_sorted)
        return MOE_ERR_NULL;
    void* ws = nullptr;
    if ((s = scratch_address((hipStream_t)stream, &ws)) != MOE_OK) return s;
    return moe_expert_ffn_q4_0(x, x_dt, T, H, w_gate_up, w_down, I, E, K, expert_offsets,
                               sorted_slots, y_sorted, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

size_t moe_linear_q4_0_workspace_bytes(int64_t T, int32_t H, int32_t R, int x_dt) {
    if (T < 0 || T > (int64_t)0x7FFFFFFF || check_dim(H, MOE_MAX_I) != MOE_OK || R < 1 ||
        R > MOE_MAX_LINEAR_ROWS || !dtype_ok(x_dt))
        return 0;
    // [0, 256): offsets {0, T}; then the slot list 0..T-1; then, on the MFMA
    // path, the activations in MFMA block order with their block sums
    size_t b = 256 + round_up((size_t)T * 4, 256);
    if (moe::linear_use_mfma(x_dt, T, H, R)) b += moe::linear_mfma_ws_bytes(T, H);
    return b;
}

moe_status moe_linear_q4_0(const void* x, int x_dt, int64_t T, int32_t H, const void* W,
                           int32_t R, float* y, void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || T > (int64_t)0x7FFFFFFF || R < 1 || R > MOE_MAX_LINEAR_ROWS) return MOE_ERR_SHAPE;
    moe_status s = check_dim(H, MOE_MAX_I);
    if (s != MOE_OK) return s;
    if (!dtype_ok(x_dt)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!x || !W || !y) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(y)) return MOE_ERR_ALIGN;
    const size_t need = moe_linear_q4_0_workspace_bytes(T, H, R, x_dt);
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    int32_t* offsets = (int32_t*)ws;
    int32_t* slots = (int32_t*)((uint8_t*)ws + 256);
    if ((s = hip_status(moe::launch_dense_index(T, offsets, slots, st))) != MOE_OK) return s;
    if (moe::linear_use_mfma(x_dt, T, H, R))
        return hip_status(moe::launch_linear_mfma(x, T, H, (const uint8_t*)W, R, offsets, slots,
                                                  (uint8_t*)ws + 256 + round_up((size_t)T * 4, 256),
                                                  y, st));
    return hip_status(moe::launch_linear_gemv(x, x_dt, T, H, (const uint8_t*)W, R, offsets, slots,
                                              y, st));
}

moe_status moe_combine(const float* y_sorted, const int32_t* slot_pos, const int32_t* topk_ids,
                       const float* topk_w, const float* expert_scale, int64_t T, int32_t K,
                       int32_t H, const void* residual, int residual_dt, float* out_f32,
                       void* out_act, int out_dt, void* stream) {
    if (T < 0 || T > (int64_t)0x7FFFFFFF || K < 1 || K > MOE_MAX_K ||
        T * (int64_t)K > (int64_t)0x7FFFFFFF)
        return MOE_ERR_SHAPE;
    moe_status s = check_dim(H, MOE_MAX_H);
    if (s != MOE_OK) return s;
    if (!dtype_ok(out_dt) || (residual && !dtype_ok(residual_dt))) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_sorted || !slot_pos || !topk_w || (expert_scale && !topk_ids) || (!out_f32 && !out_act))
        return MOE_ERR_NULL;
    if (!aligned16(y_sorted) || !aligned16(slot_pos) || !aligned16(topk_w) ||
        (topk_ids && !aligned16(topk_ids)) || (expert_scale && !aligned16(expert_scale)) ||
        (residual && !aligned16(residual)) || (out_f32 && !aligned16(out_f32)) ||
        (out_act && !aligned16(out_act)))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_combine(y_sorted, slot_pos, topk_ids, topk_w, expert_scale, T, K,
                                          H, residual, residual_dt, out_f32, out_act, out_dt,
                                          (hipStream_t)stream));
}

moe_status moe_rmsnorm(const void* x, int x_dt, const float* w, float eps, int64_t T, int32_t H,
                       void* out, int out_dt, void* stream) {
    if (T < 0 || T > (int64_t)0x7FFFFFFF) return MOE_ERR_SHAPE;
    moe_status s = check_dim(H, MOE_MAX_H);
    if (s != MOE_OK) return s;
    if (!dtype_ok(x_dt) || !dtype_ok(out_dt)) return MOE_ERR_UNSUPPORTED;
    if (!(eps >= 0.f)) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !w || !out) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return MOE_ERR_ALIGN;
    return hip_status(moe::launch_rmsnorm(x, x_dt, w, eps, T, H, out, out_dt, (hipStream_t)stream));
}

}  // extern "C"
