// Weighted combine of the routed experts' outputs, and the RMSNorm that
// precedes each layer of a stack, gfx950.
//
// Model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision, NInfer
// v3 artifact", table "What is inside": expert scales and norms are FP32.
#include "kernels.h"

namespace moe {

// out[t, o] = sum_k (w[t,k] * scale[e_k]) * y[slot_pos[t*K+k], o], fixed k order.
// Workgroup (t, b): token t, outputs 4*(256*b + thread) .. +3.  The K weights,
// scales and row positions are uniform loads; all K rows' loads are issued
// before the first product (KB >= K rows, clamped to a valid k), so a
// workgroup costs two dependent memory round trips whatever K is.
template <int RDT, int ODT, int KB>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ scale, int K, int H,
                                                      const void* __restrict__ residual,
                                                      float* __restrict__ out_f32,
                                                      void* __restrict__ out_act) {
    const int64_t t = blockIdx.x;
    const int H4 = H >> 2;
    const int j4 = min((int)(blockIdx.y * blockDim.x + threadIdx.x), H4 - 1);
    float c[KB];
    int64_t row[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int64_t s = t * K + min(k, K - 1);
        c[k] = w[s] * (scale ? scale[ids[s]] : 1.f);
        row[k] = (int64_t)slot_pos[s] * H4;
    }
    float4 v[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) v[k] = reinterpret_cast<const float4*>(y)[row[k] + j4];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        if (k < K) {
            acc.x = fmaf(c[k], v[k].x, acc.x);
            acc.y = fmaf(c[k], v[k].y, acc.y);
            acc.z = fmaf(c[k], v[k].z, acc.z);
            acc.w = fmaf(c[k], v[k].w, acc.w);
        }
    }
    if ((int)(blockIdx.y * blockDim.x + threadIdx.x) >= H4) return;
    const int64_t o = t * H + 4 * j4;
    if (out_f32) *reinterpret_cast<float4*>(out_f32 + o) = acc;
    if (out_act) {
        float r[4] = {acc.x, acc.y, acc.z, acc.w};
        if (residual) {
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] += load_act(residual, RDT, o + i);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) store_act(out_act, ODT, o + i, r[i]);
    }
}

hipError_t launch_combine(const float* y, const int32_t* slot_pos, const int32_t* ids,
                          const float* w, const float* scale, int64_t T, int K, int H,
                          const void* residual, int rdt, float* out_f32, void* out_act, int odt,
                          hipStream_t st) {
    const int threads = H >= 1024 ? 256 : 64;
    dim3 grid((unsigned)T, (unsigned)((H / 4 + threads - 1) / threads));
#define MOE_COMB(R, O)                                                                          \
    (K <= 8 ? combine_kernel<R, O, 8><<<grid, threads, 0, st>>>(y, slot_pos, ids, w, scale, K, H, \
                                                                residual, out_f32, out_act)     \
            : combine_kernel<R, O, MOE_MAX_K><<<grid, threads, 0, st>>>(                        \
                  y, slot_pos, ids, w, scale, K, H, residual, out_f32, out_act))
    if (rdt == MOE_F32 && odt == MOE_F32) MOE_COMB(MOE_F32, MOE_F32);
    else if (rdt == MOE_F32) MOE_COMB(MOE_F32, MOE_BF16);
    else if (odt == MOE_F32) MOE_COMB(MOE_BF16, MOE_F32);
    else MOE_COMB(MOE_BF16, MOE_BF16);
#undef MOE_COMB
    return hipGetLastError();
}

// out[t,:] = x[t,:] * (mean x^2 + eps)^-1/2 * w, fp32, rounded to out dtype.
template <int XDT, int ODT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x,
                                                      const float* __restrict__ wt, float eps,
                                                      int H, void* __restrict__ out) {
    const int64_t t = blockIdx.x;
    __shared__ float part[4];
    float ss = 0.f;
    for (int j = threadIdx.x; j < H; j += 256) {
        const float v = load_act(x, XDT, t * H + j);
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    for (int j = threadIdx.x; j < H; j += 256) {
        const float v = load_act(x, XDT, t * H + j);
        store_act(out, ODT, t * H + j, (v * r) * wt[j]);
    }
}

hipError_t launch_rmsnorm(const void* x, int xdt, const float* w, float eps, int64_t T, int H,
                          void* out, int odt, hipStream_t st) {
    dim3 grid((unsigned)T);
#define MOE_RMS(X, O) rmsnorm_kernel<X, O><<<grid, 256, 0, st>>>(x, w, eps, H, out)
    if (xdt == MOE_F32 && odt == MOE_F32) MOE_RMS(MOE_F32, MOE_F32);
    else if (xdt == MOE_F32) MOE_RMS(MOE_F32, MOE_BF16);
    else if (odt == MOE_F32) MOE_RMS(MOE_BF16, MOE_F32);
    else MOE_RMS(MOE_BF16, MOE_BF16);
#undef MOE_RMS
    return hipGetLastError();
}

}  // namespace moe
