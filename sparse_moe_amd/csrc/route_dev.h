// Device helpers shared by the routing kernels (router top-K, permutation).
#pragma once

#include "kernels.h"

namespace moe {

MOE_DEV uint64_t lanemask_lt() {
    const int l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// mask of the lanes of this wave whose key equals mine (keys < 512)
MOE_DEV uint64_t match_key9(uint32_t key) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const uint32_t bit = (key >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// Exclusive scan of cnt[0..n) (n <= 256) into out[0..n], out[n] = total, by 256 threads.
MOE_DEV void block_exclusive_scan256(const int* cnt, int n, int* tmp, int32_t* out_global,
                                     int* out_lds) {
    const int tid = threadIdx.x;
    int v = tid < n ? cnt[tid] : 0;
    tmp[tid] = v;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int a = tid >= d ? tmp[tid - d] : 0;
        __syncthreads();
        tmp[tid] += a;
        __syncthreads();
    }
    const int incl = tmp[tid];
    if (tid < n) {
        if (out_global) out_global[tid] = incl - v;
        if (out_lds) out_lds[tid] = incl - v;
    }
    if (tid == n - 1) {
        if (out_global) out_global[n] = incl;
        if (out_lds) out_lds[n] = incl;
    }
    __syncthreads();
}


// Stable counting sort of N <= PERM_TILE slots by one workgroup of 256 threads
// (4 rounds of 256 slots): stable ranks from the wave match plus per-wave
// counts, then offsets by a block scan, then the scatter.
MOE_DEV void permute_block(const int32_t* ids, int N, int E, int32_t* offsets,
                           int32_t* sorted_slots, int32_t* slot_pos) {
    __shared__ int run[MOE_MAX_E];
    __shared__ int wcnt[4][MOE_MAX_E];
    __shared__ int tmp[256];
    __shared__ int off[MOE_MAX_E + 1];
    const int tid = threadIdx.x, wave = tid >> 6;
    run[tid] = 0;  // blockDim == MOE_MAX_E
    int rank[PERM_TILE / 256], ex[PERM_TILE / 256];
    const int rounds = (N + 255) / 256;  // <= PERM_TILE / 256
#pragma unroll
    for (int r = 0; r < PERM_TILE / 256; ++r) {
        if (r >= rounds) break;
        const int s = r * 256 + tid;
        const bool valid = s < N;
        const int e = valid ? ids[s] : 0;
        const uint32_t key = valid ? (uint32_t)e : 256u;
#pragma unroll
        for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
        __syncthreads();
        const uint64_t m = match_key9(key);
        const int rw = __popcll(m & lanemask_lt());
        if (valid && rw == 0) wcnt[wave][e] = __popcll(m);
        __syncthreads();
        int rk = rw;
        if (valid) {
            rk += run[e];
            for (int w = 0; w < wave; ++w) rk += wcnt[w][e];
        }
        rank[r] = rk;
        ex[r] = valid ? e : -1;
        __syncthreads();
        run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        __syncthreads();
    }
    block_exclusive_scan256(run, E, tmp, offsets, off);
#pragma unroll
    for (int r = 0; r < PERM_TILE / 256; ++r) {
        if (r >= rounds) break;
        const int s = r * 256 + tid;
        if (ex[r] >= 0) {
            const int pos = off[ex[r]] + rank[r];
            sorted_slots[pos] = s;
            slot_pos[s] = pos;
        }
    }
}

// The same sort for N <= 64 slots by one wave (the caller's wave 0 alone; no
// workgroup barrier): an LDS histogram of the expert ids, an exclusive scan of
// it across the wave (lane l holds experts 4l .. 4l+3), and the stable rank of
// each slot among the slots of its expert from the wave match.
constexpr int PERM_WAVE = 64;

MOE_DEV void permute_wave(const int32_t* ids, int N, int E, int32_t* offsets,
                          int32_t* sorted_slots, int32_t* slot_pos) {
    __shared__ int hcnt[MOE_MAX_E];
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) hcnt[4 * lane + i] = 0;
    const bool valid = lane < N;
    const int e = valid ? ids[lane] : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid) atomicAdd(&hcnt[e], 1);
    __builtin_amdgcn_wave_barrier();
    int c[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i] = 4 * lane + i < E ? hcnt[4 * lane + i] : 0;
        tot += c[i];
    }
    int incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    int run = incl - tot;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ex = 4 * lane + i;
        if (ex < E) {
            offsets[ex] = run;
            hcnt[ex] = run;  // now the exclusive offsets
        }
        if (ex == E - 1) offsets[E] = run + c[i];
        run += c[i];
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t m = match_key9(valid ? (uint32_t)e : 256u);
    if (valid) {
        const int pos = hcnt[e] + __popcll(m & lanemask_lt());
        sorted_slots[pos] = lane;
        slot_pos[lane] = pos;
    }
}

// Top-K of one token's E logits by one wave; lane l holds experts l, l+64,
// l+128, l+192.  Each of the K rounds takes the wave maximum (DPP) of the
// untaken logits and the lowest expert index holding it (ballots), so equal
// logits go in ascending expert order.  Weights: softmax over the K kept
// logits.  Every lane of the wave must be active.
// COH: the logits were written by other workgroups of this launch (coherent loads).
// (all four loads unconditional, clamped to expert E-1, so that they are in
// flight together; a load in a branch waits for itself)
template <bool COH = false>
MOE_DEV void topk_load(const float* l, int E, float (&v)[4]) {
    const int lane = threadIdx.x & 63;
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        r[i] = COH ? coherent_load(l + e) : l[e];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = lane + 64 * i < E ? r[i] : 0.f;
}

// Order-preserving map of a float to an int key (v + 0 has turned -0 into +0):
// the rounds below compare keys with integer max, which the DPP steps take as
// one instruction each (a float max canonicalises its inputs first).  NaN ranks
// below every number, as under fmaxf; a taken or absent expert is INT_MIN.
MOE_DEV int topk_key(float v) {
    const int b = __float_as_int(v);
    return v != v ? INT_MIN + 1 : (b ^ ((b >> 31) & 0x7FFFFFFF));
}
MOE_DEV float topk_unkey(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// DPP move without an `old` operand (lanes without a source lane read 0): the
// compiler folds it into the min or max that consumes it.
template <int CTRL>
MOE_DEV int dpp_mov_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Wave-wide minimum and maximum, read from lane 63.  The two row broadcasts
// write every row: rows 1 and 3 take lane 15 of the row before (row 0's lanes
// read 0 and row 2's mix rows 1 and 2; neither reaches lane 63), then rows 2
// and 3 take lane 31, which holds the extremum of rows 0 and 1.

MOE_DEV int wave_min_i32(int v) {
    v = min(v, dpp_mov_i32<DPP_QUAD_XOR1>(v));
    v = min(v, dpp_mov_i32<DPP_QUAD_XOR2>(v));
    v = min(v, dpp_mov_i32<DPP_ROW_HALF_MIRROR>(v));
    v = min(v, dpp_mov_i32<DPP_ROW_MIRROR>(v));
    v = min(v, dpp_mov_i32<DPP_ROW_BCAST15>(v));
    v = min(v, dpp_mov_i32<DPP_ROW_BCAST31>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

MOE_DEV int wave_max_i32(int v) {
    v = max(v, dpp_mov_i32<DPP_QUAD_XOR1>(v));
    v = max(v, dpp_mov_i32<DPP_QUAD_XOR2>(v));
    v = max(v, dpp_mov_i32<DPP_ROW_HALF_MIRROR>(v));
    v = max(v, dpp_mov_i32<DPP_ROW_MIRROR>(v));
    v = max(v, dpp_mov_i32<DPP_ROW_BCAST15>(v));
    v = max(v, dpp_mov_i32<DPP_ROW_BCAST31>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// NT tokens at once (one wave): the K rounds of the tokens are interleaved so
// that their dependent DPP reductions overlap; each token's operations are
// those of a single-token selection.
template <int NT>
MOE_DEV void topk_select_n(const float (&lv)[NT][4], int E, int K, int32_t* const (&ids)[NT],
                           float* const (&w)[NT]) {
    const int lane = threadIdx.x & 63;
    int key[NT][4];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            key[n][i] = lane + 64 * i < E ? topk_key(lv[n][i] + 0.f) : INT_MIN;
    float selv[NT][MOE_MAX_K];
    int seli[NT][MOE_MAX_K];
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            selv[n][k] = 0.f;
            seli[n][k] = 0;
        }
        if (k < K) {
            // the maximum key, then the lowest expert index holding it: two wave
            // reductions on the vector unit (no ballot and scalar search)
            int m[NT], idx[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n)
                m[n] = wave_max_i32(max(max(key[n][0], key[n][1]), max(key[n][2], key[n][3])));
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                int li = INT_MAX;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    li = min(li, key[n][i] == m[n] ? 64 * i + lane : INT_MAX);
                idx[n] = wave_min_i32(li);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                selv[n][k] = topk_unkey(m[n]);
                seli[n][k] = idx[n];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    key[n][i] = 64 * i + lane == idx[n] ? INT_MIN : key[n][i];
            }
        }
    }
    // softmax over the K kept logits: lane k takes exp(v_k - v_0), the sum is a
    // 16-lane reduction (K <= 16) in a fixed order
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        float myv = 0.f;
        int myi = 0;
#pragma unroll
        for (int k = 0; k < MOE_MAX_K; ++k)
            if (k == lane) {
                myv = selv[n][k];
                myi = seli[n][k];
            }
        const float ex = lane < K ? expf(myv - selv[n][0]) : 0.f;
        const float s = group_sum<16>(ex);
        if (lane < K) {
            ids[n][lane] = myi;
            w[n][lane] = ex / s;
        }
    }
}

// Routing of ONE token by one wave, for latency: the same K rounds of a wave
// arg-max as topk_select (the largest key by DPP reductions; the lowest expert
// holding it by ballots, as a first set bit, instead of a second reduction),
// recording the round in which each expert is taken; then the permutation of
// the token's K slots from the set of kept experts: expert e's offset is the
// number of kept experts below e (a masked bit count), which is also the sorted
// position of the slot that took it.  Same ids, weights and permutation as
// topk_select and permute_wave, bit for bit.  ids, w, offsets, sorted_slots
// and slot_pos may point to LDS or global memory.  Every lane of the wave must
// be active.  COH: the logits were written by other workgroups of this launch.
template <bool COH>
MOE_DEV void route_one_token(const float* logits, int E, int K, int32_t* ids, float* w,
                             int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos) {
    const int lane = threadIdx.x & 63;
    float v[4];
    topk_load<COH>(logits, E, v);
    int key[4], rk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        key[i] = lane + 64 * i < E ? topk_key(v[i] + 0.f) : INT_MIN;
        rk[i] = -1;
    }
    float selv[MOE_MAX_K];
    int seli[MOE_MAX_K];
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k) {
        selv[k] = 0.f;
        seli[k] = 0;
        if (k < K) {
            const int m = wave_max_i32(max(max(key[0], key[1]), max(key[2], key[3])));
            // the lowest expert holding m: experts 64 i + lane, so the first key
            // register with a match, then its first lane
            uint64_t b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i] = __ballot(key[i] == m);
            const int idx = b[0] ? __builtin_ctzll(b[0])
                          : b[1] ? 64 + __builtin_ctzll(b[1])
                          : b[2] ? 128 + __builtin_ctzll(b[2])
                                 : 192 + __builtin_ctzll(b[3]);
            selv[k] = topk_unkey(m);
            seli[k] = idx;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool taken = 64 * i + lane == idx;
                key[i] = taken ? INT_MIN : key[i];
                rk[i] = taken ? k : rk[i];
            }
        }
    }
    // softmax over the K kept logits (topk_select_n's arithmetic)
    float myv = 0.f;
    int myi = 0;
#pragma unroll
    for (int k = 0; k < MOE_MAX_K; ++k)
        if (k == lane) {
            myv = selv[k];
            myi = seli[k];
        }
    const float ex = lane < K ? expf(myv - selv[0]) : 0.f;
    const float s = group_sum<16>(ex);
    if (lane < K) {
        ids[lane] = myi;
        w[lane] = ex / s;
    }
    // permutation: slot k (taken in round k) of expert e sits at offsets[e]
    int below = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint64_t kept = __ballot(rk[i] >= 0);
        const int off = below + (int)__builtin_amdgcn_mbcnt_hi(
                                    (uint32_t)(kept >> 32),
                                    __builtin_amdgcn_mbcnt_lo((uint32_t)kept, 0u));
        const int e = lane + 64 * i;
        if (e < E) offsets[e] = off;
        if (rk[i] >= 0) {
            sorted_slots[off] = rk[i];
            slot_pos[rk[i]] = off;
        }
        below += __popcll(kept);
    }
    if (lane == 0) offsets[E] = below;
}

MOE_DEV void topk_select(const float (&lv)[4], int E, int K, int32_t* ids, float* w) {
    const float (&l1)[1][4] = *reinterpret_cast<const float (*)[1][4]>(&lv);
    int32_t* const i1[1] = {ids};
    float* const w1[1] = {w};
    topk_select_n<1>(l1, E, K, i1, w1);
}

template <bool COH = false>
MOE_DEV void topk_token(const float* l, int E, int K, int32_t* ids, float* w) {
    float v[4];
    topk_load<COH>(l, E, v);
    topk_select(v, E, K, ids, w);
}

}  // namespace moe
