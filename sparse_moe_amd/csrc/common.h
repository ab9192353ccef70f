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

// ---- device-coherent accesses ------------------------------------------------------
// Data passed between workgroups of one launch goes through agent-scope relaxed
// atomic stores and loads, whose scope bits make the hardware keep them
// coherent across the vector L1 and the XCDs' separate L2s.  The producer waits until its stores are
// acknowledged (s_waitcnt vmcnt(0)) and then bumps a counter with a relaxed
// atomic; the consumer issues its coherent loads only after it has seen the
// final count.  Neither side needs an L2 write-back or invalidate, which an
// agent-scope release or acquire would issue (microseconds each when many
// workgroups issue one).
MOE_DEV void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV float coherent_load(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV void coherent_store_act(void* p, int dt, int64_t i, float v) {
    if (dt == MOE_F32)
        coherent_store((float*)p + i, v);
    else
        __hip_atomic_store((uint16_t*)p + i, (uint16_t)f32_to_bf16(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV uint64_t coherent_load_u64(const void* p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// ---- workgroup barrier ordering LDS only ------------------------------------------
// __syncthreads() fences all memory, which makes the compiler drain every
// outstanding global load (vmcnt(0)) at each barrier and defeats prefetching
// into registers.  Staged LDS tiles only need LDS ordering: a workgroup-scope
// fence on the local address space waits for LDS (lgkmcnt) alone.
MOE_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- GELU with the tanh approximation ----------------------------------------
// 0.5 z (1 + tanh(a)) = z / (1 + exp(-2a)), a = sqrt(2/pi) (z + 0.044715 z^3);
// exp through the hardware exp2.
MOE_DEV float gelu_tanh(float z) {
    const float c2 = 2.0f * 0.7978845608028654f * 1.4426950408889634f;  // 2 sqrt(2/pi) log2(e)
    const float a = c2 * fmaf(0.044715f * z, z * z, z);
    return z / (1.0f + exp2f(-a));
}

// ---- wave64 reductions through DPP (no LDS round trips) --------------------------
// update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl): lanes whose row is
// masked off keep `old`.
template <int CTRL, int ROW_MASK = 0xF>
MOE_DEV float dpp_f32(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xF, false));
}

constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// DPP move without an `old` operand (lanes without a source lane read 0), so
// no register has to be prepared for the lanes it does not write.
template <int CTRL>
MOE_DEV float dpp_mov_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G a power of two <= 64).  The result is
// valid in lane G-1 of each group (and in every lane of the group for G <= 16;
// for G >= 32 the other lanes hold partial sums).  Every lane of the wave must
// be active.
template <int G>
MOE_DEV float group_sum(float v) {
    if (G >= 2) v += dpp_mov_f32<DPP_QUAD_XOR1>(v);
    if (G >= 4) v += dpp_mov_f32<DPP_QUAD_XOR2>(v);
    if (G >= 8) v += dpp_mov_f32<DPP_ROW_HALF_MIRROR>(v);
    if (G >= 16) v += dpp_mov_f32<DPP_ROW_MIRROR>(v);
    // lane 15 of each row onto the next row: rows 1 and 3 then hold the sums
    // of lanes 0-31 and 32-63 (rows 0 and 2 are not used)
    if (G >= 32) v += dpp_mov_f32<DPP_ROW_BCAST15>(v);
    // lane 31 onto rows 2 and 3: lane 63 holds the sum of all 64 lanes
    if (G >= 64) v += dpp_mov_f32<DPP_ROW_BCAST31>(v);
    return v;
}

// Maximum over the whole wave, returned uniformly (read from lane 63).
MOE_DEV float wave_max(float v) {
    v = fmaxf(v, dpp_f32<DPP_QUAD_XOR1>(v, v));
    v = fmaxf(v, dpp_f32<DPP_QUAD_XOR2>(v, v));
    v = fmaxf(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v, v));
    v = fmaxf(v, dpp_f32<DPP_ROW_MIRROR>(v, v));
    v = fmaxf(v, dpp_f32<DPP_ROW_BCAST15, 0xA>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<DPP_ROW_BCAST31, 0xC>(-INFINITY, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

MOE_DEV float wave_sum(float v) {
    v = group_sum<64>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

MOE_DEV int lane_id() { return __lane_id(); }
