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
// One workgroup per token; a thread holds chunks c and c + 256 of 8 consecutive
// elements (H <= 4096) in registers, so the row is read once, with 16-byte
// loads, and written with 16-byte stores.
template <int XDT>
MOE_DEV void load8(const void* x, int64_t e0, float v[8]) {
    if (XDT == MOE_F32) {
        const float4 a = *reinterpret_cast<const float4*>((const float*)x + e0);
        const float4 b = *reinterpret_cast<const float4*>((const float*)x + e0 + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>((const uint16_t*)x + e0);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}

template <int ODT>
MOE_DEV void store8(void* out, int64_t e0, const float v[8]) {
    if (ODT == MOE_F32) {
        *reinterpret_cast<float4*>((float*)out + e0) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>((float*)out + e0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>((uint16_t*)out + e0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int XDT, int ODT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x,
                                                      const float* __restrict__ wt, float eps,
                                                      int H, void* __restrict__ out) {
    const int64_t t = blockIdx.x;
    __shared__ float part[4];
    const int nch = H >> 3;
    float v[2][8];
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c = threadIdx.x + 256 * r;
        if (c < nch) {
            load8<XDT>(x, t * H + 8 * c, v[r]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(v[r][i], v[r][i], ss);
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float rs = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int c = threadIdx.x + 256 * r;
        if (c < nch) {
            const float4 w0 = *reinterpret_cast<const float4*>(wt + 8 * c);
            const float4 w1 = *reinterpret_cast<const float4*>(wt + 8 * c + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (v[r][i] * rs) * wv[i];
            store8<ODT>(out, t * H + 8 * c, o);
        }
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
