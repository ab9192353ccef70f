// Launchers of the gfx950 kernels (internal; the public ABI is sparse_moe.h).
#pragma once

#include "common.h"

namespace moe {

constexpr int ROUTER_GEMV_MAX_T = 8;   // router: tokens per workgroup of the per-expert GEMV (T < 64)
constexpr int ROUTER_MFMA_MIN_T = 64;  // router: bf16 MFMA (exact three-way weight split) from here
constexpr int PERM_TILE = 1024;        // permutation: slots per tile (256 threads x 4)
constexpr int DIGIT_NMAX = 30583;       // largest |n| with 4 balanced base-16 digits: 7*(1+16+256+4096)
constexpr int FFN_MFMA_MIN_T = 64;     // expert FFN: bf16 MFMA grouped GEMM from this many tokens

// The one-token decode's completion counters: DECODE_CTR_LINES ints, one per
// 256-byte line (int index DECODE_CTR_STRIDE * j), so that the increments of
// many workgroups and the polls spread over several memory channels; int 1 is
// the timeout flag.  The header takes DECODE_CTR_BYTES of the workspace.
constexpr int DECODE_CTR_LINES = 64;
constexpr int DECODE_CTR_STRIDE = 64;
constexpr size_t DECODE_CTR_BYTES = DECODE_CTR_LINES * DECODE_CTR_STRIDE * sizeof(int);
// int index of the i-th word to clear, i < DECODE_CTR_LINES + 1
__host__ __device__ inline int decode_ctr_word(int i) { return i < DECODE_CTR_LINES ? DECODE_CTR_STRIDE * i : 1; }

// zero_ctr (optional): a decode counter header that the launch clears (zeroed
// by the router launch of the same call)
hipError_t launch_router_logits(const void* x, int x_dt, int64_t T, int H, const float* W,
                                const float* rsc, const float* bias, int E, float* logits,
                                hipStream_t st, int* zero_ctr = nullptr);
hipError_t launch_zero_decode_ctr(int* p, hipStream_t st);
hipError_t launch_route_small(const void* x, int x_dt, int T, int H, const float* W,
                              const float* rsc, const float* bias, int E, int K, float* logits,
                              int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_slots,
                              int32_t* slot_pos, int* counter, hipStream_t st);
hipError_t launch_topk(const float* logits, int64_t T, int E, int K, int32_t* ids, float* w,
                       hipStream_t st);

size_t permute_ws_bytes(int64_t N, int E);
hipError_t launch_permute(const int32_t* ids, int N, int E, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_pos, void* ws, hipStream_t st);

hipError_t launch_ffn_gemv(const void* x, int x_dt, int64_t T, int H, const uint8_t* w_gate_up,
                           const uint8_t* w_down, int I, int E, int K, int N,
                           const int32_t* offsets, const int32_t* sorted_slots, void* h_ws,
                           float* y_sorted, hipStream_t st);

// one decode layer (router logits, gate/up with the routing inside, down with
// the combine inside): up to ROUTER_GEMV_MAX_T tokens and 64 slots, rows of an
// even number of Q4_0 blocks.  ctr: two ints, zero on entry (the one-token
// one-launch path's completion counter and timeout flag)
bool decode_layer_supported(int64_t T, int H, int I, int K);
hipError_t launch_decode_layer(const void* x, int x_dt, int T, int H, const float* logits, int E,
                               int K, const uint8_t* w_gate_up, const uint8_t* w_down, int I,
                               const float* scale, int32_t* ids, float* w, int32_t* off,
                               int32_t* ss, int32_t* sp, const void* residual, int rdt,
                               float* out_f32, void* out_act, int odt, void* h_ws, int* ctr,
                               hipStream_t st);

// bf16 activations, enough tokens, and rows of an even number of Q4_0 blocks
// (every block pair dword aligned)
inline bool ffn_use_mfma(int x_dt, int64_t T, int H, int I) {
    return x_dt == MOE_BF16 && T >= FFN_MFMA_MIN_T && H % 64 == 0 && I % 64 == 0;
}
size_t ffn_mfma_ws_bytes(int64_t T, int H, int I, int64_t N);
hipError_t launch_ffn_mfma(const void* x, int64_t T, int H, const uint8_t* w_gate_up,
                           const uint8_t* w_down, int I, int E, int K, int N,
                           const int32_t* offsets, const int32_t* sorted_slots, void* ws,
                           float* y_sorted, hipStream_t st);

// plain Q4_0 linear layer y [T, R] = x [T, H] W^T on the down-product kernels
inline bool linear_use_mfma(int x_dt, int64_t T, int H, int R) {
    return x_dt == MOE_BF16 && T >= FFN_MFMA_MIN_T && H % 64 == 0 && R % 16 == 0;
}
hipError_t launch_dense_index(int64_t T, int32_t* offsets, int32_t* slots, hipStream_t st);
hipError_t launch_linear_gemv(const void* x, int x_dt, int64_t T, int H, const uint8_t* W, int R,
                              const int32_t* offsets, const int32_t* slots, float* y,
                              hipStream_t st);
size_t linear_mfma_ws_bytes(int64_t T, int H);
hipError_t launch_linear_mfma(const void* x, int64_t T, int H, const uint8_t* W, int R,
                              const int32_t* offsets, const int32_t* slots, void* ws, float* y,
                              hipStream_t st);

hipError_t launch_combine(const float* y, const int32_t* slot_pos, const int32_t* ids,
                          const float* w, const float* scale, int64_t T, int K, int H,
                          const void* residual, int rdt, float* out_f32, void* out_act, int odt,
                          hipStream_t st);
hipError_t launch_rmsnorm(const void* x, int xdt, const float* w, float eps, int64_t T, int H,
                          void* out, int odt, hipStream_t st);

}  // namespace moe
