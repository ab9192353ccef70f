// Expert FFN for few tokens per expert (decode): Q4_0 weights streamed once
// from HBM and multiplied in place, gfx950.
//
// The model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision,
// NInfer v3 artifact" keeps the release's ggml Q4_0 blocks byte for byte and
// multiplies them in place; table "What is inside": experts are expert-major,
// a [gate; up] parent of 2 x I rows and a down matrix of H rows.
//
// Products without dequantisation: the 4-bit codes q of a block are used as
// they are stored.  XOR 0x8 turns each nibble q into the signed 4-bit value
// q - 8, and v_dot8_i32_i4 multiplies 8 of them at once with 8 signed 4-bit
// digits of the activations.  Activations are written per 32-element block as
// a fixed-point integer n_j = rint(v_j * 30583 / max|v|) (|n_j| <= 30583) in
// four balanced base-16 digits (each in [-8, 7]); the block's integer dot
// sum_j (q_j - 8) n_j is therefore exact, and the block contributes
// d * (max|v| / 30583) * dot.  The only approximation is the 15-bit fixed
// point of the activations (|error| <= max|v| / 61166 per element).
//
// Lane layout: a lane owns a pair of consecutive blocks (36 bytes, always
// 4-byte aligned) at the same position of every row it visits, so the lane's
// activation digits stay in registers; a row is covered by LPR lanes (a power
// of two >= blocks/2), a wave covers 64/LPR rows per step, and the loads of a
// wave are contiguous.
#include "kernels.h"

namespace moe {

// ---- activation digits -------------------------------------------------------
// Word (m, k) (m = qs dword 0..3, k = digit 0..3) holds digit k of the 8
// elements that the 8 nibbles of qs dword m encode: nibble p <-> element
// 4m + (p >> 1) + 16 (p & 1).
template <int ADT>
MOE_DEV void quantize_block32(const void* src, int64_t e0, uint32_t* words, float* scale) {
    float v[32];
    if (ADT == MOE_F32) {
        const float4* p = reinterpret_cast<const float4*>((const float*)src + e0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 q = p[i];
            v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
        }
    } else {
        const uint4* p = reinterpret_cast<const uint4*>((const uint16_t*)src + e0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 q = p[i];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    uint32_t wd[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wd[i] = 0;
    float s = 0.f;
    if (amax > 0.f) {
        const float inv = (float)DIGIT_NMAX / amax;
        s = amax / (float)DIGIT_NMAX;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            int n = (int)rintf(v[j] * inv);
            n = max(-DIGIT_NMAX, min(DIGIT_NMAX, n));
            const int m = (j & 15) >> 2;
            const int p = ((j & 3) << 1) | (j >> 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int d = ((n + 8) & 15) - 8;
                wd[m * 4 + k] |= (uint32_t)(d & 15) << (4 * p);
                n = (n - d) >> 4;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) words[i] = wd[i];
    *scale = s;
}

// signed 4-bit codes (q - 8) of one Q4_0 block times the 4 digit words of each
// qs dword: exact integer sum_j (q_j - 8) n_j
MOE_DEV int block_idot(const uint32_t q[4], const uint32_t* x16) {
    int d0 = 0, d1 = 0, d2 = 0, d3 = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int qm = (int)(q[m] ^ 0x88888888u);
        d0 = __builtin_amdgcn_sdot8(qm, (int)x16[4 * m + 0], d0, false);
        d1 = __builtin_amdgcn_sdot8(qm, (int)x16[4 * m + 1], d1, false);
        d2 = __builtin_amdgcn_sdot8(qm, (int)x16[4 * m + 2], d2, false);
        d3 = __builtin_amdgcn_sdot8(qm, (int)x16[4 * m + 3], d3, false);
    }
    return d0 + (d1 << 4) + (d2 << 8) + (d3 << 12);
}

// Scales and qs dwords of a block pair: block A at bytes 0..17, block B at
// bytes 18..35 of the lane's 36-byte window (always 4-byte aligned).  nh = how
// many of the two blocks exist (the last pair of a row with an odd block count
// has one: only its 18 bytes are read).  Missing blocks get a zero scale.
struct PairDec {
    float dA, dB;
    uint32_t qA[4], qB[4];
};

MOE_DEV PairDec load_pair(const uint8_t* p, int nh) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    u32x4a4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    uint32_t w8 = 0u, tail = 0u;
    if (nh >= 1) a = __builtin_nontemporal_load(reinterpret_cast<const u32x4a4*>(q));
    if (nh == 2) {
        b = __builtin_nontemporal_load(reinterpret_cast<const u32x4a4*>(q + 4));
        w8 = __builtin_nontemporal_load(q + 8);
    } else if (nh == 1) {
        tail = *reinterpret_cast<const uint16_t*>(p + 16);
    }
    const uint32_t w4 = (nh == 2) ? b.x : tail;
    PairDec r;
    r.dA = f16_bits_to_f32(a.x);
    r.dB = f16_bits_to_f32(w4 >> 16);
    r.qA[0] = __builtin_amdgcn_perm(a.y, a.x, 0x05040302u);
    r.qA[1] = __builtin_amdgcn_perm(a.z, a.y, 0x05040302u);
    r.qA[2] = __builtin_amdgcn_perm(a.w, a.z, 0x05040302u);
    r.qA[3] = __builtin_amdgcn_perm(w4, a.w, 0x05040302u);
    r.qB[0] = b.y;
    r.qB[1] = b.z;
    r.qB[2] = b.w;
    r.qB[3] = w8;
    return r;
}

// ---- kernel --------------------------------------------------------------------
// MODE 0: gate/up rows of the [gate; up] parent -> h = GELU_tanh(g) * u (act dtype)
// MODE 1: down rows -> y (fp32)
// One workgroup = 4 waves; each wave owns UPW units; a unit is RPS = 64/LPR
// output rows (MODE 0: RPS gate rows and the RPS matching up rows).
// The weights of the wave's units are loaded once into registers; tokens of
// the expert are then processed in chunks of TC.
template <int MODE, int ADT, int LPR, int TC, int UPW>
__global__ __launch_bounds__(256) void ffn_gemv_q4_0(
    const uint8_t* __restrict__ W, int nb, int I, int H, const void* __restrict__ act,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots, int K, int E,
    void* __restrict__ out) {
    constexpr int RPS = 64 / LPR;
    constexpr int NR = (MODE == 0) ? 2 : 1;  // rows per unit and lane (gate + up)
    extern __shared__ uint32_t lds[];        // [TC][nb][16] digit words, then [TC][nb] scales
    __shared__ int s_e, s_wcnt[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // -- which expert: the blockIdx.y-th expert with at least one slot
    {
        const int e = tid;
        const bool ne = e < E && offsets[e + 1] > offsets[e];
        const uint64_t b = __ballot(ne);
        if (tid == 0) s_e = -1;
        if (lane == 0) s_wcnt[wave] = __popcll(b);
        __syncthreads();
        int before = __popcll(b & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        for (int w = 0; w < wave; ++w) before += s_wcnt[w];
        if (ne && before == (int)blockIdx.y) s_e = e;
        __syncthreads();
    }
    const int e = s_e;
    if (e < 0) return;
    const int p0 = offsets[e], ne_tok = offsets[e + 1] - p0;

    const int rows_out = (MODE == 0) ? I : H;            // outputs per expert
    const int rows_tot = (MODE == 0) ? 2 * I : H;        // stored rows per expert
    const int64_t row_bytes = (int64_t)nb * 18;
    const uint8_t* We = W + (int64_t)e * rows_tot * row_bytes;
    const int g = lane / LPR, q = lane % LPR;
    const int nblk_here = min(2, max(0, nb - 2 * q));
    const int unit0 = (blockIdx.x * 4 + wave) * UPW;

    // -- weights of this wave's units: loaded once
    PairDec wt[UPW][NR];
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const int row = (unit0 + u) * RPS + g;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int srow = row + r * I;
            const int nh = row < rows_out ? nblk_here : 0;
            wt[u][r] = load_pair(We + srow * row_bytes + 36 * q, nh);
        }
    }

    uint32_t* dig = lds;
    float* dsc = reinterpret_cast<float*>(lds + TC * nb * 16);
    const int in_len = (MODE == 0) ? H : I;
    for (int c0 = 0; c0 < ne_tok; c0 += TC) {
        // -- digits of the chunk's activation rows into LDS
        __syncthreads();
        for (int task = tid; task < TC * nb; task += 256) {
            const int t = task / nb, b = task % nb;
            const int p = p0 + c0 + t;
            if (c0 + t < ne_tok) {
                const int64_t src_row = (MODE == 0) ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
                quantize_block32<ADT>(act, src_row * in_len + b * 32, dig + (t * nb + b) * 16,
                                      dsc + t * nb + b);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) dig[(t * nb + b) * 16 + i] = 0;
                dsc[t * nb + b] = 0.f;
            }
        }
        __syncthreads();
        float acc[UPW][NR][TC];
#pragma unroll
        for (int u = 0; u < UPW; ++u)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int t = 0; t < TC; ++t) acc[u][r][t] = 0.f;
        if (nblk_here > 0) {
#pragma unroll
            for (int t = 0; t < TC; ++t) {
                uint32_t xa[16], xb[16];
                const uint32_t* da = dig + (t * nb + 2 * q) * 16;
#pragma unroll
                for (int i = 0; i < 16; ++i) xa[i] = da[i];
                const float sa = dsc[t * nb + 2 * q];
                float sb = 0.f;
                if (nblk_here == 2) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) xb[i] = da[16 + i];
                    sb = dsc[t * nb + 2 * q + 1];
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) xb[i] = 0;
                }
#pragma unroll
                for (int u = 0; u < UPW; ++u)
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const int ia = block_idot(wt[u][r].qA, xa);
                        const int ib = block_idot(wt[u][r].qB, xb);
                        acc[u][r][t] = fmaf(wt[u][r].dA * sa, (float)ia, acc[u][r][t]);
                        acc[u][r][t] = fmaf(wt[u][r].dB * sb, (float)ib, acc[u][r][t]);
                    }
            }
        }
        // -- reduce over the LPR lanes of a row, write
#pragma unroll
        for (int u = 0; u < UPW; ++u) {
            const int row = (unit0 + u) * RPS + g;
#pragma unroll
            for (int t = 0; t < TC; ++t) {
                float v[NR];
#pragma unroll
                for (int r = 0; r < NR; ++r) v[r] = group_sum<LPR>(acc[u][r][t]);
                if (q == 0 && row < rows_out && c0 + t < ne_tok) {
                    const int64_t p = p0 + c0 + t;
                    if (MODE == 0) {
                        store_act(out, ADT, p * I + row, gelu_tanh(v[0]) * v[NR - 1]);
                    } else {
                        reinterpret_cast<float*>(out)[p * H + row] = v[0];
                    }
                }
            }
        }
    }
}

// ---- dispatch ---------------------------------------------------------------------
template <int MODE, int ADT, int LPR>
static void launch_mode(const uint8_t* W, int nb, int I, int H, const void* act,
                        const int32_t* offsets, const int32_t* sorted_slots, int K, int E,
                        int n_active, void* out, hipStream_t st) {
    constexpr int TC = 2, UPW = 4, RPS = 64 / LPR;
    const int rows_out = (MODE == 0) ? I : H;
    const int units = (rows_out + RPS - 1) / RPS;
    const int wgs = (units + 4 * UPW - 1) / (4 * UPW);
    const size_t lds = (size_t)TC * nb * 17 * sizeof(uint32_t);
    dim3 grid(wgs, n_active);
    ffn_gemv_q4_0<MODE, ADT, LPR, TC, UPW><<<grid, 256, lds, st>>>(W, nb, I, H, act, offsets,
                                                                   sorted_slots, K, E, out);
}

template <int MODE, int ADT>
static void launch_lpr(const uint8_t* W, int nb, int I, int H, const void* act,
                       const int32_t* offsets, const int32_t* sorted_slots, int K, int E,
                       int n_active, void* out, hipStream_t st) {
    const int pairs = (nb + 1) / 2;
#define MOE_LPR_CASE(L)                                                                        \
    if (pairs <= L) {                                                                          \
        launch_mode<MODE, ADT, L>(W, nb, I, H, act, offsets, sorted_slots, K, E, n_active, out, \
                                  st);                                                         \
        return;                                                                                \
    }
    MOE_LPR_CASE(1) MOE_LPR_CASE(2) MOE_LPR_CASE(4) MOE_LPR_CASE(8) MOE_LPR_CASE(16)
    MOE_LPR_CASE(32) MOE_LPR_CASE(64)
#undef MOE_LPR_CASE
}

hipError_t launch_ffn_gemv(const void* x, int x_dt, int H, const uint8_t* w_gate_up,
                           const uint8_t* w_down, int I, int E, int K, int N,
                           const int32_t* offsets, const int32_t* sorted_slots, void* h_ws,
                           float* y_sorted, hipStream_t st) {
    const int n_active = min(E, N);
    if (x_dt == MOE_F32) {
        launch_lpr<0, MOE_F32>(w_gate_up, H / 32, I, H, x, offsets, sorted_slots, K, E, n_active,
                               h_ws, st);
        launch_lpr<1, MOE_F32>(w_down, I / 32, I, H, h_ws, offsets, sorted_slots, K, E, n_active,
                               y_sorted, st);
    } else {
        launch_lpr<0, MOE_BF16>(w_gate_up, H / 32, I, H, x, offsets, sorted_slots, K, E, n_active,
                                h_ws, st);
        launch_lpr<1, MOE_BF16>(w_down, I / 32, I, H, h_ws, offsets, sorted_slots, K, E, n_active,
                                y_sorted, st);
    }
    return hipGetLastError();
}

}  // namespace moe
