// Internal helpers shared by the gfx950 kernels of the routed-MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_moe.h"

#define MOE_DEV static __device__ __forceinline__

typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 ------------------------------------------------------------------
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
MOE_DEV uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

MOE_DEV float load_act(const void* p, int dt, int64_t i) {
    return dt == MOE_F32 ? ((const float*)p)[i] : bf16_to_f32(((const uint16_t*)p)[i]);
}

MOE_DEV void store_act(void* p, int dt, int64_t i, float v) {
    if (dt == MOE_F32)
        ((float*)p)[i] = v;
    else
        ((uint16_t*)p)[i] = f32_to_bf16(v);
}

// ---- fp16 scale of a Q4_0 block --------------------------------------------
MOE_DEV float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// ---- GELU with the tanh approximation ----------------------------------------
MOE_DEV float gelu_tanh(float z) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}

// ---- wave64 reductions --------------------------------------------------------
MOE_DEV float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// sum over aligned groups of G lanes (G a power of two <= 64); every lane of a
// group receives the group's sum
template <int G>
MOE_DEV float group_sum(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

MOE_DEV int lane_id() { return __lane_id(); }
