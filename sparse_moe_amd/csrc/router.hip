// Router logits (FP32) and top-K with renormalised softmax weights, gfx950.
//
// Model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision, NInfer
// v3 artifact", table "What is inside": the router and router scale are FP32.
// Each token keeps the K largest logits (descending; equal logits in ascending
// expert order) with softmax weights over the K kept logits.
#include <type_traits>

#include "route_dev.h"

namespace moe {

// ---------------------------------------------------------------------------
// Few tokens: one workgroup per expert streams its W_r row once (float4 loads,
// all issued at once) and dots it with up to ROUTER_GEMV_MAX_T tokens.
constexpr int ROUTER_MAX_CHUNKS = MOE_MAX_H / 256;  // float4 chunks of 64 lanes per row

// One expert per workgroup: wave w takes a quarter of the float4 chunks of the
// expert's W_r row, dots them with every token and leaves its per-token partial
// sums in part[w][t].  Every load (W_r, router scale, the TT token rows) is
// issued before the first product: the loads are unconditional, at clamped
// chunk and token indices, so they go out together instead of one round trip
// each.  Each token's products and sums are the same for any TT >= T.
template <int XDT, int TT, bool RSC>
MOE_DEV void expert_partials(const void* __restrict__ x, int T, int H, const float* __restrict__ W,
                             const float* __restrict__ rsc, int e,
                             float (*part)[ROUTER_GEMV_MAX_T]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H4 = H >> 2, nch = (H4 + 63) >> 6;
    const int c0 = wave * nch / 4, c1 = (wave + 1) * nch / 4;
    const float4* wr = reinterpret_cast<const float4*>(W + (int64_t)e * H);
    constexpr int CPW = ROUTER_MAX_CHUNKS / 4;
    int j4[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = max(0, min(c0 + i, c1 - 1));  // a valid chunk even past this wave's range
        j4[i] = min(lane + 64 * c, H4 - 1);
    }
    float4 wv[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) wv[i] = wr[j4[i]];
    float4 sv[RSC ? CPW : 1];
    if constexpr (RSC) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) sv[i] = reinterpret_cast<const float4*>(rsc)[j4[i]];
    }
    using XV = typename std::conditional<XDT == MOE_F32, float4, uint2>::type;
    XV xr[CPW][TT];
#pragma unroll
    for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int t = 0; t < TT; ++t)
            xr[i][t] = reinterpret_cast<const XV*>(x)[(int64_t)min(t, T - 1) * H4 + j4[i]];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int c = c0 + i;
        if (RSC) {
            wv[i].x *= sv[i].x; wv[i].y *= sv[i].y; wv[i].z *= sv[i].z; wv[i].w *= sv[i].w;
        }
        if (c >= c1 || lane + 64 * c >= H4) wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        if (c0 + i < c1) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                if (t < T) {
                    float4 xv;
                    if constexpr (XDT == MOE_F32) {
                        xv = xr[i][t];
                    } else {
                        const uint2 b = xr[i][t];
                        xv = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                                         __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
                    }
                    acc[t] = fmaf(xv.x, wv[i].x, acc[t]);
                    acc[t] = fmaf(xv.y, wv[i].y, acc[t]);
                    acc[t] = fmaf(xv.z, wv[i].z, acc[t]);
                    acc[t] = fmaf(xv.w, wv[i].w, acc[t]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        if (t < T) {
            const float sum = wave_sum(acc[t]);
            if (lane == 0) part[wave][t] = sum;
        }
    }
}

// Workgroup (e, g): expert e for tokens 8g .. 8g+7.  A token's logit is the same
// sequence of operations whatever T is and wherever the token sits in the batch
// (the fused few-token kernel uses the same expert_partials and final sum), so
// every T below ROUTER_MFMA_MIN_T routes a token exactly as T = 1 does.
template <int XDT, int TT, bool RSC>
__global__ __launch_bounds__(256) void router_logits_gemv(const void* __restrict__ x, int T, int H,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ rsc,
                                                          const float* __restrict__ bias, int E,
                                                          float* __restrict__ logits,
                                                          int* __restrict__ zero_ctr) {
    __shared__ float part[4][ROUTER_GEMV_MAX_T];
    const int e = blockIdx.x;
    if (zero_ctr && e == 0 && blockIdx.y == 0 && threadIdx.x <= DECODE_CTR_LINES)
        zero_ctr[decode_ctr_word(threadIdx.x)] = 0;
    const int t0 = blockIdx.y * ROUTER_GEMV_MAX_T, tg = min(ROUTER_GEMV_MAX_T, T - t0);
    const void* xg = XDT == MOE_F32 ? (const void*)((const float*)x + (int64_t)t0 * H)
                                    : (const void*)((const uint16_t*)x + (int64_t)t0 * H);
    expert_partials<XDT, TT, RSC>(xg, tg, H, W, rsc, e, part);
    __syncthreads();
    const int t = threadIdx.x;
    if (t < tg)
        logits[(int64_t)(t0 + t) * E + e] =
            ((part[0][t] + part[1][t]) + (part[2][t] + part[3][t])) + (bias ? bias[e] : 0.f);
}

// ---------------------------------------------------------------------------
// Many tokens (fp32 activations, or an expert count that is not a multiple of
// 32): 32 tokens x 64 experts per workgroup, K-tiles of 32 staged in LDS.
constexpr int RT_BM = 32, RT_BN = 64, RT_BK = 32;

template <int XDT>
__global__ __launch_bounds__(256) void router_logits_tiled(const void* __restrict__ x, int T, int H,
                                                           const float* __restrict__ W,
                                                           const float* __restrict__ rsc,
                                                           const float* __restrict__ bias, int E,
                                                           float* __restrict__ logits) {
    __shared__ float As[RT_BK][RT_BM + 4];
    __shared__ float Bs[RT_BK][RT_BN + 4];
    const int tid = threadIdx.x;
    const int m0 = blockIdx.x * RT_BM, n0 = blockIdx.y * RT_BN;
    const int tx = tid & 15, ty = tid >> 4;  // experts tx*4.., tokens ty*2..
    float acc[2][4] = {};
    for (int k0 = 0; k0 < H; k0 += RT_BK) {
        {   // x tile: 32 tokens x 32 k, 4 consecutive k per thread
            const int m = tid >> 3, k4 = (tid & 7) * 4;
            const int tok = m0 + m;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (tok < T) {
                const int64_t off = (int64_t)tok * H + k0 + k4;
                if (XDT == MOE_F32) {
                    const float4 q = *reinterpret_cast<const float4*>((const float*)x + off);
                    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
                } else {
                    const uint2 b = *reinterpret_cast<const uint2*>((const uint16_t*)x + off);
                    v[0] = __uint_as_float(b.x << 16); v[1] = __uint_as_float(b.x & 0xFFFF0000u);
                    v[2] = __uint_as_float(b.y << 16); v[3] = __uint_as_float(b.y & 0xFFFF0000u);
                }
                if (rsc) {
                    const float4 s = *reinterpret_cast<const float4*>(rsc + k0 + k4);
                    v[0] *= s.x; v[1] *= s.y; v[2] *= s.z; v[3] *= s.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) As[k4 + i][m] = v[i];
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {  // W tile: 64 experts x 32 k
            const int n = (tid >> 3) + 32 * r, k4 = (tid & 7) * 4;
            float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
            if (n0 + n < E) q = *reinterpret_cast<const float4*>(W + (int64_t)(n0 + n) * H + k0 + k4);
            Bs[k4 + 0][n] = q.x; Bs[k4 + 1][n] = q.y; Bs[k4 + 2][n] = q.z; Bs[k4 + 3][n] = q.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < RT_BK; ++k) {
            const float a0 = As[k][ty * 2], a1 = As[k][ty * 2 + 1];
            const float4 b = *reinterpret_cast<const float4*>(&Bs[k][tx * 4]);
            acc[0][0] += a0 * b.x; acc[0][1] += a0 * b.y; acc[0][2] += a0 * b.z; acc[0][3] += a0 * b.w;
            acc[1][0] += a1 * b.x; acc[1][1] += a1 * b.y; acc[1][2] += a1 * b.z; acc[1][3] += a1 * b.w;
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tok = m0 + ty * 2 + i;
        if (tok >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = n0 + tx * 4 + j;
            if (e < E) logits[(int64_t)tok * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
        }
    }
}

// ---- top-K: one wave per token ---------------------------------------------
__global__ __launch_bounds__(256) void topk_softmax(const float* __restrict__ logits, int64_t T,
                                                    int E, int K, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token(logits + t * E, E, K, ids + t * K, w + t * K);
}



// Few tokens, routing fused into one kernel: the router GEMV by every
// workgroup (one expert each, logits written with coherent stores), then
// the last workgroup to finish (counted with an agent-scope atomic in the
// workspace) runs top-K for every token on coherently loaded logits and the
// permutation of the T*K slots, and resets the counter to zero.
template <int XDT, int TT, bool RSC>
__global__ __launch_bounds__(256) void route_small(const void* __restrict__ x, int T, int H,
                                                   const float* __restrict__ W,
                                                   const float* __restrict__ rsc,
                                                   const float* __restrict__ bias, int E, int K,
                                                   float* __restrict__ logits,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted_slots,
                                                   int32_t* __restrict__ slot_pos,
                                                   int* __restrict__ counter) {
    const int wave = threadIdx.x >> 6;
    __shared__ float part[4][ROUTER_GEMV_MAX_T];
    const int e = blockIdx.x;  // one expert per workgroup, H split over its waves
    expert_partials<XDT, TT, RSC>(x, T, H, W, rsc, e, part);
    __syncthreads();
    {
        const int t = threadIdx.x;
        if (t < T)
            coherent_store(logits + (int64_t)t * E + e,
                           ((part[0][t] + part[1][t]) + (part[2][t] + part[3][t])) +
                               (bias ? bias[e] : 0.f));
    }
    __shared__ int s_last;
    // The logits are stored by threads t < T <= 8, all in wave 0, which also
    // makes the count: the wave waits until its coherent stores are
    // acknowledged, then increments; the last workgroup reads them with
    // coherent loads issued after its increment has returned.  No L2
    // write-back or invalidate is needed on either side.
    if (threadIdx.x < 64) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (int)gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (T == 1) {  // one token: one wave, short dependency chains
        if (wave == 0) route_one_token<true>(logits, E, K, ids, w, offsets, sorted_slots, slot_pos);
        if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // wave w takes tokens w and w + 4 (both selections interleaved)
    const int t0 = wave, t1 = wave + 4;
    if (t1 < T) {
        float v[2][4];
        topk_load<true>(logits + (int64_t)t0 * E, E, v[0]);
        topk_load<true>(logits + (int64_t)t1 * E, E, v[1]);
        int32_t* const ip[2] = {ids + t0 * K, ids + t1 * K};
        float* const wp[2] = {w + t0 * K, w + t1 * K};
        topk_select_n<2>(v, E, K, ip, wp);
    } else if (t0 < T) {
        float v[4];
        topk_load<true>(logits + (int64_t)t0 * E, E, v);
        topk_select(v, E, K, ids + t0 * K, w + t0 * K);
    }
    __syncthreads();  // ids of every token are written
    if (T * K <= PERM_WAVE) {
        if (wave == 0) permute_wave(ids, T * K, E, offsets, sorted_slots, slot_pos);
    } else {
        permute_block(ids, T * K, E, offsets, sorted_slots, slot_pos);
    }
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// token-count bucket (1, 2, 4 or 8 rows loaded per chunk) and router-scale
// presence, as template arguments
template <class F>
static void router_variant(int x_dt, int T, bool rsc, F&& f) {
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    auto with_t = [&](auto xdt, auto r) {
        if (T <= 1) f(xdt, I1{}, r);
        else if (T <= 2) f(xdt, I2{}, r);
        else if (T <= 4) f(xdt, I4{}, r);
        else f(xdt, I8{}, r);
    };
    auto with_r = [&](auto xdt) { rsc ? with_t(xdt, std::true_type{}) : with_t(xdt, std::false_type{}); };
    if (x_dt == MOE_F32) with_r(std::integral_constant<int, MOE_F32>{});
    else with_r(std::integral_constant<int, MOE_BF16>{});
}

hipError_t launch_route_small(const void* x, int x_dt, int T, int H, const float* W,
                              const float* rsc, const float* bias, int E, int K, float* logits,
                              int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_slots,
                              int32_t* slot_pos, int* counter, hipStream_t st) {
    router_variant(x_dt, T, rsc != nullptr, [&](auto xdt, auto tt, auto r) {
        route_small<decltype(xdt)::value, decltype(tt)::value, decltype(r)::value>
            <<<dim3(E), 256, 0, st>>>(x, T, H, W, rsc, bias, E, K, logits, ids, w, offsets,
                                      sorted_slots, slot_pos, counter);
    });
    return hipGetLastError();
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Many tokens, bf16 activations: logits on bf16 MFMA (v_mfma_f32_16x16x32_bf16).
// Each fp32 router weight (times the router scale, when given) is split by bit
// truncation into three bf16 parts hi + mid + lo that add up to it exactly (the
// top 8, next 8 and last 8 significant bits of fp32's 24), so
// x W = x hi + x mid + x lo: exact products, fp32 accumulation, three MFMAs per
// K step.  Workgroup tile: 32 tokens x 32 experts (each weight fragment and its
// split serve two token fragments); its 4 waves take a quarter of H each and
// add their partial sums through LDS in a fixed order.
typedef __attribute__((ext_vector_type(8))) __bf16 rbf16x8;
typedef uint32_t ru32x4 __attribute__((ext_vector_type(4)));

MOE_DEV f32x4 rmfma(ru32x4 a, ru32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rbf16x8, a),
                                                   __builtin_bit_cast(rbf16x8, b), c, 0, 0, 0);
}

// 8 fp32 weights -> their hi, mid and lo bf16 parts, packed in k order
MOE_DEV void split3(const float (&w)[8], ru32x4& hi, ru32x4& mid, ru32x4& lo) {
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t u = __float_as_uint(w[j]);
        h[j] = u & 0xFFFF0000u;
        const float r1 = w[j] - __uint_as_float(h[j]);       // exact
        m[j] = __float_as_uint(r1) & 0xFFFF0000u;
        const float r2 = r1 - __uint_as_float(m[j]);          // exact, at most 8 significant bits
        l[j] = __float_as_uint(r2) & 0xFFFF0000u;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        hi[q] = (h[2 * q] >> 16) | h[2 * q + 1];
        mid[q] = (m[2 * q] >> 16) | m[2 * q + 1];
        lo[q] = (l[2 * q] >> 16) | l[2 * q + 1];
    }
}

// tokens from which the bf16 router runs ROUTER_WIDE_TF 16-token fragments per
// workgroup (each split weight fragment then serves more MFMAs)
constexpr int ROUTER_WIDE_MIN_T = 2048;
constexpr int ROUTER_WIDE_TF = 4;

// NW waves split K; TF fragments of 16 tokens per workgroup share each split
// weight fragment (the split is VALU work, so more token fragments per split
// means fewer operations per MFMA, at the cost of fewer workgroups).
template <int NW, int TF, bool RSC>
__global__ __launch_bounds__(NW * 64) void router_logits_mfma(const uint16_t* __restrict__ x, int T, int H,
                                                          const float* __restrict__ W,
                                                          const float* __restrict__ rsc,
                                                          const float* __restrict__ bias, int E,
                                                          float* __restrict__ logits) {
    __shared__ f32x4 part[NW - 1][TF][2][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int t0 = blockIdx.x * (16 * TF);
    const int e0 = blockIdx.y * 32;
    // this wave's share of H (H is a multiple of 32)
    const int nsteps = H >> 5;
    const int k_begin = (nsteps * wave / NW) * 32, k_end = (nsteps * (wave + 1) / NW) * 32;
    // A operand: lane (token row l16 of fragment f, k group g); B operand: lane
    // (expert column l16, k group g)
    const uint16_t* xf[TF];
#pragma unroll
    for (int f = 0; f < TF; ++f) xf[f] = x + (int64_t)min(t0 + 16 * f + l16, T - 1) * H + 8 * g;
    const float* w0 = W + (int64_t)(e0 + l16) * H + 8 * g;
    const float* w1 = W + (int64_t)(e0 + 16 + l16) * H + 8 * g;
    f32x4 acc[TF][2];
#pragma unroll
    for (int f = 0; f < TF; ++f) acc[f][0] = acc[f][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // the loads of step k+32 are issued before the MFMAs of step k (clamped at the end)
    struct Step {
        ru32x4 a[TF];
        float4 p0, p1, q0, q1;
        float4 s0[RSC ? 1 : 0], s1[RSC ? 1 : 0];
    };
    auto load = [&](Step& S, int k) {
#pragma unroll
        for (int f = 0; f < TF; ++f) S.a[f] = *(const ru32x4*)(xf[f] + k);
        S.p0 = *(const float4*)(w0 + k);
        S.p1 = *(const float4*)(w0 + k + 4);
        S.q0 = *(const float4*)(w1 + k);
        S.q1 = *(const float4*)(w1 + k + 4);
        if constexpr (RSC) {
            S.s0[0] = *(const float4*)(rsc + 8 * g + k);
            S.s1[0] = *(const float4*)(rsc + 8 * g + k + 4);
        }
    };
    Step cur, nxt;
    load(cur, min(k_begin, H - 32));
    for (int k = k_begin; k < k_end; k += 32) {
        load(nxt, min(k + 32, H - 32));
        float wa[8] = {cur.p0.x, cur.p0.y, cur.p0.z, cur.p0.w, cur.p1.x, cur.p1.y, cur.p1.z, cur.p1.w};
        float wb[8] = {cur.q0.x, cur.q0.y, cur.q0.z, cur.q0.w, cur.q1.x, cur.q1.y, cur.q1.z, cur.q1.w};
        if constexpr (RSC) {
            const float sv[8] = {cur.s0[0].x, cur.s0[0].y, cur.s0[0].z, cur.s0[0].w,
                                 cur.s1[0].x, cur.s1[0].y, cur.s1[0].z, cur.s1[0].w};
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                wa[jj] *= sv[jj];
                wb[jj] *= sv[jj];
            }
        }
        ru32x4 h0, m0, lo0, h1, m1, lo1;
        split3(wa, h0, m0, lo0);
        split3(wb, h1, m1, lo1);
        // hi, then mid, then lo parts: the same per-element order for every tile shape
#pragma unroll
        for (int f = 0; f < TF; ++f) {
            acc[f][0] = rmfma(cur.a[f], h0, acc[f][0]);
            acc[f][1] = rmfma(cur.a[f], h1, acc[f][1]);
        }
#pragma unroll
        for (int f = 0; f < TF; ++f) {
            acc[f][0] = rmfma(cur.a[f], m0, acc[f][0]);
            acc[f][1] = rmfma(cur.a[f], m1, acc[f][1]);
        }
#pragma unroll
        for (int f = 0; f < TF; ++f) {
            acc[f][0] = rmfma(cur.a[f], lo0, acc[f][0]);
            acc[f][1] = rmfma(cur.a[f], lo1, acc[f][1]);
        }
        cur = nxt;
    }
    // partial sums of waves 1..NW-1 to LDS; wave 0 adds them in order and stores
    if (wave > 0) {
#pragma unroll
        for (int f = 0; f < TF; ++f) {
            part[wave - 1][f][0][lane] = acc[f][0];
            part[wave - 1][f][1][lane] = acc[f][1];
        }
    }
    __syncthreads();
    if (wave > 0) return;
    // in wave order (a rolled loop: unrolled, the partial reads of many waves
    // are all hoisted and the registers run out)
#pragma unroll 1
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
        for (int f = 0; f < TF; ++f) {
            acc[f][0] += part[w][f][0][lane];
            acc[f][1] += part[w][f][1][lane];
        }
    // output lane (token rows 16 f + 4g .. +3, expert column l16)
    const float b0 = bias ? bias[e0 + l16] : 0.f, b1 = bias ? bias[e0 + 16 + l16] : 0.f;
#pragma unroll
    for (int f = 0; f < TF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * f + 4 * g + i;
            if (t < T) {
                logits[(int64_t)t * E + e0 + l16] = acc[f][0][i] + b0;
                logits[(int64_t)t * E + e0 + 16 + l16] = acc[f][1][i] + b1;
            }
        }
}

// Few tiles (a few hundred tokens): 16 tokens x 16 EF experts per workgroup
// (many workgroups: each CU's loads, not the arithmetic, set the pace), K
// split over NW waves, and each wave issues the loads of PF K steps at a time
// before their MFMAs.  Same split, same per-element order (hi, mid, lo per
// step, steps in k order, waves' partial sums in wave order).
template <int NW, int PF, int EF, bool RSC>
__global__ __launch_bounds__(NW * 64) void router_logits_mfma_batch(
    const uint16_t* __restrict__ x, int T, int H, const float* __restrict__ W,
    const float* __restrict__ rsc, const float* __restrict__ bias, int E, float* __restrict__ logits) {
    __shared__ f32x4 part[NW - 1][EF][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int t0 = blockIdx.x * 16;
    const int e0 = blockIdx.y * 16 * EF;
    const int nsteps = H >> 5;
    const int k_begin = (nsteps * wave / NW) * 32, k_end = (nsteps * (wave + 1) / NW) * 32;
    const uint16_t* xf = x + (int64_t)min(t0 + l16, T - 1) * H + 8 * g;
    const float* wp[EF];
#pragma unroll
    for (int f = 0; f < EF; ++f) wp[f] = W + (int64_t)(e0 + 16 * f + l16) * H + 8 * g;
    f32x4 acc[EF];
#pragma unroll
    for (int f = 0; f < EF; ++f) acc[f] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int kb = k_begin; kb < k_end; kb += 32 * PF) {
        ru32x4 a[PF];
        f32x4 p0[PF][EF], p1[PF][EF];
        f32x4 s0[RSC ? PF : 1], s1[RSC ? PF : 1];
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            const int k = min(kb + 32 * s, k_end - 32);  // past the end: a step that is not used
            a[s] = *(const ru32x4*)(xf + k);
#pragma unroll
            for (int f = 0; f < EF; ++f) {
                p0[s][f] = *(const f32x4*)(wp[f] + k);
                p1[s][f] = *(const f32x4*)(wp[f] + k + 4);
            }
            if constexpr (RSC) {
                s0[s] = *(const f32x4*)(rsc + 8 * g + k);
                s1[s] = *(const f32x4*)(rsc + 8 * g + k + 4);
            }
        }
        // all of the batch's loads land here (otherwise the compiler moves each
        // step's loads next to its MFMAs, one round trip per step)
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            asm volatile("" ::"v"(a[s]));
#pragma unroll
            for (int f = 0; f < EF; ++f) asm volatile("" ::"v"(p0[s][f]), "v"(p1[s][f]));
            if constexpr (RSC) asm volatile("" ::"v"(s0[s]), "v"(s1[s]));
        }
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            if (kb + 32 * s >= k_end) break;
            ru32x4 hi[EF], mid[EF], lo[EF];
#pragma unroll
            for (int f = 0; f < EF; ++f) {
                float wv[8] = {p0[s][f].x, p0[s][f].y, p0[s][f].z, p0[s][f].w,
                               p1[s][f].x, p1[s][f].y, p1[s][f].z, p1[s][f].w};
                if constexpr (RSC) {
                    const float sv[8] = {s0[s].x, s0[s].y, s0[s].z, s0[s].w,
                                         s1[s].x, s1[s].y, s1[s].z, s1[s].w};
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) wv[jj] *= sv[jj];
                }
                split3(wv, hi[f], mid[f], lo[f]);
            }
#pragma unroll
            for (int f = 0; f < EF; ++f) acc[f] = rmfma(a[s], hi[f], acc[f]);
#pragma unroll
            for (int f = 0; f < EF; ++f) acc[f] = rmfma(a[s], mid[f], acc[f]);
#pragma unroll
            for (int f = 0; f < EF; ++f) acc[f] = rmfma(a[s], lo[f], acc[f]);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int f = 0; f < EF; ++f) part[wave - 1][f][lane] = acc[f];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll 1
    for (int w = 0; w < NW - 1; ++w) {
#pragma unroll
        for (int f = 0; f < EF; ++f) acc[f] += part[w][f][lane];
    }
#pragma unroll
    for (int f = 0; f < EF; ++f) {
        const float b = bias ? bias[e0 + 16 * f + l16] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * g + i;
            if (t < T) logits[(int64_t)t * E + e0 + 16 * f + l16] = acc[f][i] + b;
        }
    }
}

__global__ void zero_decode_ctr(int* __restrict__ p) {
    if ((int)threadIdx.x <= DECODE_CTR_LINES) p[decode_ctr_word(threadIdx.x)] = 0;
}

hipError_t launch_zero_decode_ctr(int* p, hipStream_t st) {
    zero_decode_ctr<<<1, 128, 0, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, int x_dt, int64_t T, int H, const float* W,
                                const float* rsc, const float* bias, int E, float* logits,
                                hipStream_t st, int* zero_ctr) {
    // only the few-token kernel below zeroes the counter itself
    if (zero_ctr && T >= ROUTER_MFMA_MIN_T) {
        const hipError_t e = launch_zero_decode_ctr(zero_ctr, st);
        if (e != hipSuccess) return e;
    }
    if (x_dt == MOE_BF16 && T >= ROUTER_MFMA_MIN_T && E % 32 == 0) {
        // 32 tokens x 32 experts per workgroup, K split over 4 waves (over 8 when
        // the tiles are too few to fill the chip); many tokens: ROUTER_WIDE_TF
        // token fragments per workgroup, K over 8 waves
        const int64_t tiles32 = (T + 31) / 32 * (E / 32);
        auto go = [&](auto rsc_c) {
            constexpr bool R = decltype(rsc_c)::value;
            if (T >= ROUTER_WIDE_MIN_T) {
                constexpr int TF = ROUTER_WIDE_TF;
                dim3 grid((unsigned)((T + 16 * TF - 1) / (16 * TF)), E / 32);
                router_logits_mfma<4, TF, R><<<grid, 256, 0, st>>>((const uint16_t*)x, (int)T, H, W,
                                                                   rsc, bias, E, logits);
            } else if (tiles32 <= 128) {
                // few tiles: 16 tokens x 16 experts per workgroup, K over 8 waves,
                // each wave's loads issued in batches of 11 steps (all of its
                // steps for H = 2,816; 6 with the router scale, whose loads take
                // registers too)
                constexpr int PF = R ? 6 : 11;
                dim3 grid((unsigned)((T + 15) / 16), E / 16);
                router_logits_mfma_batch<8, PF, 1, R><<<grid, 512, 0, st>>>((const uint16_t*)x, (int)T, H,
                                                                            W, rsc, bias, E, logits);
            } else {
                dim3 grid((unsigned)((T + 31) / 32), E / 32);
                router_logits_mfma<4, 2, R><<<grid, 256, 0, st>>>((const uint16_t*)x, (int)T, H, W,
                                                                  rsc, bias, E, logits);
            }
        };
        if (rsc) go(std::true_type{}); else go(std::false_type{});
    } else if (T < ROUTER_MFMA_MIN_T) {
        dim3 grid(E, (unsigned)((T + ROUTER_GEMV_MAX_T - 1) / ROUTER_GEMV_MAX_T));
        router_variant(x_dt, (int)T, rsc != nullptr, [&](auto xdt, auto tt, auto r) {
            router_logits_gemv<decltype(xdt)::value, decltype(tt)::value, decltype(r)::value>
                <<<grid, 256, 0, st>>>(x, (int)T, H, W, rsc, bias, E, logits, zero_ctr);
        });
    } else {
        dim3 grid((unsigned)((T + RT_BM - 1) / RT_BM), (E + RT_BN - 1) / RT_BN);
        if (x_dt == MOE_F32)
            router_logits_tiled<MOE_F32><<<grid, 256, 0, st>>>(x, (int)T, H, W, rsc, bias, E, logits);
        else
            router_logits_tiled<MOE_BF16><<<grid, 256, 0, st>>>(x, (int)T, H, W, rsc, bias, E, logits);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int K, int32_t* ids, float* w,
                       hipStream_t st) {
    dim3 grid((unsigned)((T + 3) / 4));
    topk_softmax<<<grid, 256, 0, st>>>(logits, T, E, K, ids, w);
    return hipGetLastError();
}

}  // namespace moe
