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
// point of the activations (|error| <= max|v| / 61166 per element, max|v| the
// largest magnitude of the element's 32-element block); it applies to fp32 and
// bf16 activations alike, and to the hidden h of the down product.  A block
// whose largest magnitude is below the fp32 normal range keeps that bound only
// as far as its scale max|v| / 30583 is representable.
//
// Lane layout: a lane owns a pair of consecutive blocks (36 bytes, always
// 4-byte aligned) at the same position of every row it visits, so the lane's
// activation digits stay in registers; a row is covered by LPR lanes (a power
// of two >= blocks/2), a wave covers 64/LPR rows per step, and the loads of a
// wave are contiguous.
#include <algorithm>
#include <type_traits>

#include "route_dev.h"

namespace moe {

// ---- activation digits -------------------------------------------------------
// Word (m, k) (m = qs dword 0..3, k = digit 0..3) holds digit k of the 8
// elements that the 8 nibbles of qs dword m encode: nibble p <-> element
// 4m + (p >> 1) + 16 (p & 1).  In LDS, word i (= 4m + k) of block b of token
// slot t sits at dig[(t * 16 + i) * nbp + b] (nbp = blocks rounded up to even),
// so lanes reading the 2 blocks of their pair read consecutive 8-byte words.
// A quad of lanes digitises one 32-element block:
// lane m of the quad owns elements 4m..4m+3 and 4m+16..4m+19, so it produces
// the 4 words of qs dword m; the block maximum comes from a quad reduction.
// Every lane of a quad must be active.
// COH: agent-scope relaxed 8-byte loads, for data another workgroup of the
// same launch stored with agent-scope stores (coherent across the L2 slices)
template <int ADT, bool COH = false>
MOE_DEV void load_quarter(const void* src, int64_t e0, int m, float v[8]) {
    if (COH) {
        uint64_t u[4];
        if (ADT == MOE_F32) {
            const float* f = (const float*)src + e0 + 4 * m;
            u[0] = coherent_load_u64(f); u[1] = coherent_load_u64(f + 2);
            u[2] = coherent_load_u64(f + 16); u[3] = coherent_load_u64(f + 18);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = __uint_as_float((uint32_t)u[j]);
                v[2 * j + 1] = __uint_as_float((uint32_t)(u[j] >> 32));
            }
        } else {
            const uint16_t* s = (const uint16_t*)src + e0 + 4 * m;
            u[0] = coherent_load_u64(s); u[1] = coherent_load_u64(s + 16);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t lo = (uint32_t)u[j], hi = (uint32_t)(u[j] >> 32);
                v[4 * j] = __uint_as_float(lo << 16); v[4 * j + 1] = __uint_as_float(lo & 0xFFFF0000u);
                v[4 * j + 2] = __uint_as_float(hi << 16); v[4 * j + 3] = __uint_as_float(hi & 0xFFFF0000u);
            }
        }
    } else if (ADT == MOE_F32) {
        const float4 lo = reinterpret_cast<const float4*>((const float*)src + e0 + 4 * m)[0];
        const float4 hi = reinterpret_cast<const float4*>((const float*)src + e0 + 16 + 4 * m)[0];
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    } else {
        const uint2 lo = reinterpret_cast<const uint2*>((const uint16_t*)src + e0 + 4 * m)[0];
        const uint2 hi = reinterpret_cast<const uint2*>((const uint16_t*)src + e0 + 16 + 4 * m)[0];
        v[0] = __uint_as_float(lo.x << 16); v[1] = __uint_as_float(lo.x & 0xFFFF0000u);
        v[2] = __uint_as_float(lo.y << 16); v[3] = __uint_as_float(lo.y & 0xFFFF0000u);
        v[4] = __uint_as_float(hi.x << 16); v[5] = __uint_as_float(hi.x & 0xFFFF0000u);
        v[6] = __uint_as_float(hi.y << 16); v[7] = __uint_as_float(hi.y & 0xFFFF0000u);
    }
}

MOE_DEV void digitize_quarter(const float v[8], int m, uint32_t* words, int wstride, float* scale) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, dpp_mov_f32<DPP_QUAD_XOR1>(amax));
    amax = fmaxf(amax, dpp_mov_f32<DPP_QUAD_XOR2>(amax));
    uint32_t wd[4] = {0u, 0u, 0u, 0u};
    float s = 0.f;
    if (amax > 0.f) {
        // blocks below 2^-64 are scaled up by 2^64 (exactly) first, so that
        // DIGIT_NMAX / amax stays finite down to the smallest subnormal
        const float pre = amax < 0x1p-64f ? 0x1p64f : 1.f;
        const float inv = (float)DIGIT_NMAX / (amax * pre);
        s = amax / (float)DIGIT_NMAX;
        uint32_t u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int n = (int)rintf((v[j] * pre) * inv);
            n = max(-DIGIT_NMAX, min(DIGIT_NMAX, n));
            // n + 0x8888 = sum_k h_k 16^k with hex digits h_k, so n = sum_k (h_k - 8) 16^k:
            // the balanced digits are h_k - 8, whose 4-bit two's complement is h_k ^ 8
            // (16 bits: |n| <= DIGIT_NMAX keeps n + 0x8888 below 2^16)
            u[j] = (uint32_t)(n + 0x8888) ^ 0x8888u;
        }
        // Word k takes digit k of element j at nibble p(j) = 2 (j & 3) + (j >> 2): a
        // nibble transpose.  Elements in nibble order pair up as the 16-bit halves of
        // R_i (nibbles a0..a3 b0..b3), whose nibbles are zipped to a0 b0 a1 b1 .. a3 b3
        // (a byte swap, then a nibble swap), so byte k of R_i is the pair's digit k;
        // a 4 x 4 byte transpose of R_0..R_3 then gives the words.
        uint32_t R[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // nibble positions 2i and 2i+1 hold elements i and i + 4
            uint32_t x = u[i] | (u[i + 4] << 16);
            x = __builtin_amdgcn_perm(x, x, 0x03010200u);
            R[i] = (x & 0xF00FF00Fu) | ((x >> 4) & 0x00F000F0u) | ((x << 4) & 0x0F000F00u);
        }
        const uint32_t t0 = __builtin_amdgcn_perm(R[1], R[0], 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(R[1], R[0], 0x07030602u);
        const uint32_t t2 = __builtin_amdgcn_perm(R[3], R[2], 0x05010400u);
        const uint32_t t3 = __builtin_amdgcn_perm(R[3], R[2], 0x07030602u);
        wd[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
        wd[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
        wd[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
        wd[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) words[(4 * m + k) * wstride] = wd[k];
    if (m == 0) *scale = s;
}

// signed 4-bit codes (q - 8) of one Q4_0 block times the 4 digit words of each
// qs dword: exact integer sum_j (q_j - 8) n_j.  The digit sums are combined by
// Horner's rule, each digit's dot products accumulating onto 16 times the sum
// so far (|sum| < 2^24, exact in int32): one shift per digit instead of a
// zeroed accumulator per digit and a final shift-and-add.
MOE_DEV int block_idot(const uint32_t q[4], const uint32_t* x16) {
    int qm[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qm[m] = (int)(q[m] ^ 0x88888888u);
    int d = 0;
#pragma unroll
    for (int k = 3; k >= 0; --k) {
        d <<= 4;
#pragma unroll
        for (int m = 0; m < 4; ++m) d = __builtin_amdgcn_sdot8(qm[m], (int)x16[4 * m + k], d, false);
    }
    return d;
}

// Scales and qs dwords of a block pair: block A at bytes 0..17, block B at
// bytes 18..35 of a lane's 36-byte window.  nh = how many of the two blocks
// exist (the last pair of a row with an odd block count has one); a missing
// block gets a zero scale, so its products vanish.
struct PairDec {
    float dA, dB;
    uint32_t qA[4], qB[4];
};

// window read from LDS.  EVEN_NB: rows hold an even number of blocks, so every
// window starts 4-byte aligned; otherwise read it as 2-byte halves.
template <bool EVEN_NB>
MOE_DEV PairDec lds_pair(const uint8_t* p, int nh) {
    uint32_t w[9];
    if (EVEN_NB) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int i = 0; i < 9; ++i) w[i] = q[i];
    } else {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
        for (int i = 0; i < 9; ++i) w[i] = (uint32_t)q[2 * i] | ((uint32_t)q[2 * i + 1] << 16);
    }
    PairDec d;
    d.dA = nh >= 1 ? f16_bits_to_f32(w[0]) : 0.f;
    d.dB = nh == 2 ? f16_bits_to_f32(w[4] >> 16) : 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        d.qA[m] = __builtin_amdgcn_perm(w[m + 1], w[m], 0x05040302u);
        d.qB[m] = w[5 + m];
    }
    return d;
}

// the same window already in registers (rows of an even block count)
MOE_DEV PairDec reg_pair(const uint32_t (&w)[9], int nh) {
    PairDec d;
    d.dA = nh >= 1 ? f16_bits_to_f32(w[0]) : 0.f;
    d.dB = nh == 2 ? f16_bits_to_f32(w[4] >> 16) : 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        d.qA[m] = __builtin_amdgcn_perm(w[m + 1], w[m], 0x05040302u);
        d.qB[m] = w[5 + m];
    }
    return d;
}

// Load bytes [s0, s1) of a weight matrix with coalesced 16-byte loads
// (consecutive lanes read consecutive 16 bytes) into registers; store_span then
// writes them to the wave's LDS region.  The copy starts at the 16-byte boundary
// at or below s0; the matrix base is 16-byte aligned and its size a multiple of
// 16, so no chunk leaves the matrix.  Exactly NCH loads are issued (lanes past
// the span re-read its last chunk), so the number of loads in flight is known at
// compile time and the activations, loaded earlier, can be used while these are
// still in flight.  Returns the LDS offset of byte s0.
template <int NCH>
MOE_DEV int load_span(const uint8_t* mat, int64_t s0, int64_t s1, int lane, u32x4a4 (&v)[NCH]) {
    const int64_t a0 = s0 & ~(int64_t)15;
    const int last = (int)((s1 - a0 + 15) >> 4) - 1;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = min(64 * i + lane, last);
        v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4a4*>(mat + a0 + 16 * (int64_t)c));
    }
    return (int)(s0 - a0);
}

template <int NCH>
MOE_DEV void store_span(uint8_t* lds_wave, int lane, const u32x4a4 (&v)[NCH]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        *reinterpret_cast<uint4*>(lds_wave + 1024 * i + 16 * lane) = make_uint4(v[i].x, v[i].y, v[i].z, v[i].w);
}

// steps per wave: gate/up waves cover 2 output rows (row pairs), down waves 8
constexpr int DIRECT_ROW_MULT = 2;
// (twice that with direct register windows: no LDS span to size, and the
// longer stream per workgroup pays for its fixed latency)
template <int MODE, int LPR, bool DIRECT>
constexpr int steps_per_wave() {
    constexpr int rows = ((MODE == 0) ? 2 : 8) * (DIRECT ? DIRECT_ROW_MULT : 1);
    return (64 / LPR) >= rows ? 1 : rows / (64 / LPR);
}

// ---- kernel --------------------------------------------------------------------
// MODE 0: gate/up rows of the [gate; up] parent -> h = GELU_tanh(g) * u (act dtype)
// MODE 1: down rows -> y (fp32)
// One workgroup = 4 waves.  A wave owns UPW steps of RPS = 64/LPR output rows
// (MODE 0: the gate rows and the matching up rows); it stages those rows in its
// own LDS region with coalesced loads, then lane (g, q) of a step computes block
// pair q of row g from LDS.  Tokens of the expert are processed in chunks of TC
// whose activation digits are staged in LDS once per workgroup.
// One workgroup tile: rows [bx * 4 * RPW, ...) of the by-th active expert.
// DIRECT (rows of an even block count only): every lane loads its own 36-byte
// pair windows straight into registers (two 16-byte and one 4-byte load per
// window) instead of staging the rows through LDS with coalesced loads.  The
// requests are less regular, but the workgroup needs no LDS for weights, so
// more workgroups fit on a CU and more of the stream is in flight: the better
// trade when the grid is several times the chip (many experts, few tokens).
// ONE: a single-token call, so every gate/up slot reads activation row 0 (no
// dependent read of the slot's token before the activation loads).
// One lane's share of a row's dot product: its block pair's exact integer
// products with the activation digits, scaled by d * (max|v| / 30583) per block.
MOE_DEV float pair_acc(const PairDec& w, const uint32_t* xa, const uint32_t* xb, float sa, float sb) {
    const int ia = block_idot(w.qA, xa);
    const int ib = block_idot(w.qB, xb);
    return fmaf(w.dA * sa, (float)ia, (w.dB * sb) * (float)ib);
}

// Routing prologue of gemv_tile that does nothing (the routing is an input, and
// the workgroup's expert is looked up from the offsets).  A prologue that
// routes the batch itself returns true when it also knows the workgroup's
// expert e, its first sorted slot p0 and slot count n.
struct NoRoute {
    __device__ __forceinline__ bool operator()(int, int&, int&, int&) const { return false; }
};

template <int MODE, int ADT, int LPR, int TC, int UPW, bool EVEN_NB, bool DIRECT, bool ONE,
          bool SLOT_H = false, bool COH = false, class Route = NoRoute>
MOE_DEV void gemv_tile(const uint8_t* __restrict__ W, int nb, int I, int H,
                       const void* __restrict__ act, const int32_t* offsets,
                       const int32_t* sorted_slots, int K, int E,
                       void* __restrict__ out, int wave_lds_bytes, uint8_t* smem, int bx, int by,
                       Route route = Route()) {
    constexpr int RPS = 64 / LPR;
    constexpr int RPW = RPS * UPW;           // rows (MODE 0: row pairs) per wave
    constexpr int NR = (MODE == 0) ? 2 : 1;  // spans per wave (gate, up)
    // staging loads per span: rows hold at most 2*LPR blocks (36*LPR bytes)
    constexpr int NCH = (RPW * 36 * LPR + 15 + 1023) / 1024;
    __shared__ int s_e, s_p0, s_n, s_wcnt[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const int nbp = (nb + 1) & ~1;  // blocks per activation row, rounded up to a pair
    uint32_t* dig = reinterpret_cast<uint32_t*>(smem + 4 * wave_lds_bytes);
    float* dsc = reinterpret_cast<float*>(dig + TC * 16 * nbp);
    const int in_len = (MODE == 0) ? H : I;
    constexpr int NTASK = 2 * TC;  // quarter-block tasks per thread: TC * 128 blocks * 4 / 256
    // this workgroup's expert: first slot and slot count (set by the lookup below;
    // a single-token call has one slot per expert)
    int p0 = 0, ne_tok = 1;

    // activation rows of a chunk -> registers (one quarter block per task)
    float xv[NTASK][8];
    auto load_x = [&](int c0) {
        int64_t src_row[TC];
#pragma unroll
        for (int t = 0; t < TC; ++t) {
            const int p = __builtin_amdgcn_readfirstlane(p0 + min(c0 + t, ne_tok - 1));
            src_row[t] = (MODE == 0) ? (ONE ? 0 : (int64_t)(sorted_slots[p] / K)) : (int64_t)p;
        }
#pragma unroll
        for (int i = 0; i < NTASK; ++i) {
            const int task = tid + 256 * i;
            const int m = task & 3, tb = task >> 2;
            const int t = tb / nb, b = tb % nb;
            int64_t row = src_row[0];
#pragma unroll
            for (int j = 1; j < TC; ++j)
                if (t == j) row = src_row[j];
            // unconditional (clamped) so that the count of loads in flight is static
            const bool ok = task < TC * nb * 4 && c0 + t < ne_tok;
            load_quarter<ADT>(act, ok ? row * in_len + b * 32 : 0, m, xv[i]);
        }
    };
    // registers -> activation digits in LDS
    auto digitize = [&](int c0) {
#pragma unroll
        for (int i = 0; i < NTASK; ++i) {
            const int task = tid + 256 * i;
            if (task < TC * nb * 4) {
                const int m = task & 3, tb = task >> 2;
                const int t = tb / nb, b = tb % nb;
                uint32_t* wbase = dig + (int64_t)t * 16 * nbp + b;
                if (c0 + t < ne_tok) {
                    digitize_quarter(xv[i], m, wbase, nbp, dsc + t * nbp + b);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) wbase[(4 * m + k) * nbp] = 0u;
                    if (m == 0) dsc[t * nbp + b] = 0.f;
                }
            }
        }
    };

    // the activations first, so that waiting for them does not wait for the
    // weights; the gate/up product of a single-token call reads row 0 of x
    // whatever the routing, so it issues them before the routing is known
    constexpr bool EARLY_X = ONE && MODE == 0;
    if constexpr (EARLY_X) load_x(0);
    // the routing prologue (a fused decode layer) or nothing
    int e = -1;
    if (!route(by, e, p0, ne_tok)) {
        // which expert: the by-th expert with at least one slot
        const int ex = tid;
        int o0 = 0, o1 = 0;
        if (ex < E) {
            o0 = offsets[ex];
            o1 = offsets[ex + 1];
        }
        const bool ne = o1 > o0;
        const uint64_t b = __ballot(ne);
        if (tid == 0) s_e = -1;
        if (lane == 0) s_wcnt[wave] = __popcll(b);
        __syncthreads();
        int before = __popcll(b & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        for (int w = 0; w < wave; ++w) before += s_wcnt[w];
        if (ne && before == by) {
            s_e = ex;
            s_p0 = o0;
            s_n = o1 - o0;
        }
        __syncthreads();
        e = s_e;
        if (e < 0) return;
        p0 = s_p0;
        ne_tok = s_n;
    }

    if constexpr (!EARLY_X) load_x(0);

    const int rows_out = (MODE == 0) ? I : H;            // outputs per expert
    const int rows_tot = (MODE == 0) ? 2 * I : H;        // stored rows per expert
    const int64_t row_bytes = (int64_t)nb * 18;
    const uint8_t* We = W + (int64_t)e * rows_tot * row_bytes;
    const int g = lane / LPR, q = lane % LPR;
    const int nblk_here = min(2, max(0, nb - 2 * q));
    const int row0 = (bx * 4 + wave) * RPW;              // first output row of this wave
    const int nrows = max(0, min(RPW, rows_out - row0));

    uint8_t* wl = smem + wave * wave_lds_bytes;
    const int span_bytes = NCH * 1024 - 16;

    // -- this wave's rows: all loads in flight at once (into registers)
    constexpr int NCHS = DIRECT ? 1 : NCH;
    constexpr int UD = DIRECT ? UPW : 1, ND = DIRECT ? NR : 1;
    int loff[NR];
    u32x4a4 wreg[NR][NCHS];
    uint32_t wd[UD][ND][9];
    if constexpr (DIRECT) {
        // unconditional (clamped to a valid row and pair) so that the number of
        // loads in flight is static
        const int qq = min(q, nb / 2 - 1);
#pragma unroll
        for (int u = 0; u < UPW; ++u) {
            const int lr = min(u * RPS + g, max(nrows - 1, 0));
            const int row = nrows > 0 ? row0 + lr : 0;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint8_t* p = We + (int64_t)(row + r * I) * row_bytes + 36 * qq;
                const u32x4a4 a = *reinterpret_cast<const u32x4a4*>(p);
                const u32x4a4 b = *reinterpret_cast<const u32x4a4*>(p + 16);
                const uint32_t c = *reinterpret_cast<const uint32_t*>(p + 32);
                wd[u][r][0] = a.x; wd[u][r][1] = a.y; wd[u][r][2] = a.z; wd[u][r][3] = a.w;
                wd[u][r][4] = b.x; wd[u][r][5] = b.y; wd[u][r][6] = b.z; wd[u][r][7] = b.w;
                wd[u][r][8] = c;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {  // unconditional: waves past the last row load one chunk
            const int64_t s0 = nrows > 0 ? (int64_t)(row0 + r * I) * row_bytes : 0;
            const int64_t s1 = nrows > 0 ? s0 + nrows * row_bytes : 16;
            loff[r] = load_span<NCHS>(We, s0, s1, lane, wreg[r]);
        }
    }
    if (nbp != nb) {  // the pad block of an odd block count reads as zero
        for (int i = tid; i < TC * 16; i += 256) dig[i * nbp + nb] = 0u;
        for (int i = tid; i < TC; i += 256) dsc[i * nbp + nb] = 0.f;
    }

    // products of the staged rows with the chunk's digits, reductions, outputs
    auto compute = [&](int c0) {
        if (!DIRECT && c0 == 0) {
#pragma unroll
            for (int r = 0; r < NR; ++r) store_span<NCHS>(wl + r * (span_bytes + 16), lane, wreg[r]);
        }
        __syncthreads();  // digits of every wave and this wave's rows are in LDS
        const int qp = min(q, nbp / 2 - 1);   // lanes past the row's pairs read a valid pair
        uint32_t xa[TC][16], xb[TC][16];
        float sa[TC], sb[TC];
#pragma unroll
        for (int t = 0; t < TC; ++t) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint2 v = reinterpret_cast<const uint2*>(dig + (t * 16 + i) * nbp)[qp];
                xa[t][i] = v.x;
                xb[t][i] = v.y;
            }
            const float2 sv = reinterpret_cast<const float2*>(dsc + t * nbp)[qp];
            sa[t] = sv.x;
            sb[t] = sv.y;
        }
        float res[UPW][TC][NR];
#pragma unroll
        for (int u = 0; u < UPW; ++u) {
            const int lr = u * RPS + g;           // row within the wave's span
            float acc[NR][TC];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int nh = lr < nrows ? nblk_here : 0;
                PairDec w;
                if constexpr (DIRECT) {
                    w = reg_pair(wd[u][r], nh);
                } else {
                    const int off = loff[r] + lr * (int)row_bytes + 36 * q;
                    w = lds_pair<EVEN_NB>(wl + r * (span_bytes + 16) + (nh > 0 ? off : 0), nh);
                }
#pragma unroll
                for (int t = 0; t < TC; ++t) acc[r][t] = pair_acc(w, xa[t], xb[t], sa[t], sb[t]);
            }
#pragma unroll
            for (int t = 0; t < TC; ++t)
#pragma unroll
                for (int r = 0; r < NR; ++r) res[u][t][r] = group_sum<LPR>(acc[r][t]);
        }
        if (LPR == 64) {
            // one row per step: every sum sits in lane 63; spread them so that lane
            // u*TC + t finishes (u, t) and the GELU evaluations run side by side
            float mine[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) mine[r] = 0.f;
#pragma unroll
            for (int u = 0; u < UPW; ++u)
#pragma unroll
                for (int t = 0; t < TC; ++t)
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const float v = __int_as_float(
                            __builtin_amdgcn_readlane(__float_as_int(res[u][t][r]), 63));
                        if (lane == u * TC + t) mine[r] = v;
                    }
            const int u = lane / TC, t = lane % TC;
            if (lane < UPW * TC && u < nrows && c0 + t < ne_tok) {
                const int64_t p = p0 + c0 + t;
                const int row = row0 + u;
                if (MODE == 0)
                    (COH ? coherent_store_act : store_act)(
                        out, ADT, (SLOT_H ? (int64_t)sorted_slots[p] : p) * I + row,
                        gelu_tanh(mine[0]) * mine[NR - 1]);
                else
                    reinterpret_cast<float*>(out)[p * H + row] = mine[0];
            }
        } else {
#pragma unroll
            for (int u = 0; u < UPW; ++u) {
                const int lr = u * RPS + g;
#pragma unroll
                for (int t = 0; t < TC; ++t) {
                    if (q == LPR - 1 && lr < nrows && c0 + t < ne_tok) {
                        const int64_t p = p0 + c0 + t;
                        const int row = row0 + lr;
                        if (MODE == 0)
                            (COH ? coherent_store_act : store_act)(
                                out, ADT, (SLOT_H ? (int64_t)sorted_slots[p] : p) * I + row,
                                gelu_tanh(res[u][t][0]) * res[u][t][NR - 1]);
                        else
                            reinterpret_cast<float*>(out)[p * H + row] = res[u][t][0];
                    }
                }
            }
        }
    };
    digitize(0);
    compute(0);
    for (int c0 = TC; c0 < ne_tok; c0 += TC) {
        __syncthreads();  // digits of the previous chunk are no longer read
        load_x(c0);
        digitize(c0);
        compute(c0);
    }
}

template <int MODE, int ADT, int LPR, int TC, int UPW, bool EVEN_NB, bool DIRECT, bool ONE>
__global__ __launch_bounds__(256) void ffn_gemv_q4_0(
    const uint8_t* __restrict__ W, int nb, int I, int H, const void* __restrict__ act,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_slots, int K, int E,
    void* __restrict__ out, int wave_lds_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    gemv_tile<MODE, ADT, LPR, TC, UPW, EVEN_NB, DIRECT, ONE>(W, nb, I, H, act, offsets, sorted_slots, K, E, out,
                                                wave_lds_bytes, smem, blockIdx.x, blockIdx.y);
}

// ---- dispatch ---------------------------------------------------------------------
template <int MODE, int ADT, int LPR, int TC, bool EVEN_NB, bool DIRECT, bool ONE>
static void launch_mode(const uint8_t* W, int nb, int I, int H, const void* act,
                        const int32_t* offsets, const int32_t* sorted_slots, int K, int E,
                        int n_active, void* out, hipStream_t st) {
    constexpr int RPS = 64 / LPR;
    constexpr int UPW = steps_per_wave<MODE, LPR, DIRECT>();
    constexpr int RPW = RPS * UPW;
    constexpr int NR = (MODE == 0) ? 2 : 1;
    const int rows_out = (MODE == 0) ? I : H;
    const int wgs = (rows_out + 4 * RPW - 1) / (4 * RPW);
    constexpr int NCH = (RPW * 36 * LPR + 15 + 1023) / 1024;
    const int wave_lds = DIRECT ? 0 : NR * NCH * 1024;
    const size_t lds = (size_t)4 * wave_lds + (size_t)TC * ((nb + 1) & ~1) * 17 * sizeof(uint32_t);
    dim3 grid(wgs, n_active);
    ffn_gemv_q4_0<MODE, ADT, LPR, TC, UPW, EVEN_NB, DIRECT, ONE><<<grid, 256, lds, st>>>(
        W, nb, I, H, act, offsets, sorted_slots, K, E, out, wave_lds);
}

template <int MODE, int ADT, int TC, bool DIRECT, bool ONE>
static void launch_lpr(const uint8_t* W, int nb, int I, int H, const void* act,
                       const int32_t* offsets, const int32_t* sorted_slots, int K, int E,
                       int n_active, void* out, hipStream_t st) {
    const int pairs = (nb + 1) / 2;
#define MOE_LPR_CASE(L)                                                                         \
    if (pairs <= L) {                                                                           \
        if (nb & 1)                                                                             \
            launch_mode<MODE, ADT, L, TC, false, false, ONE>(W, nb, I, H, act, offsets, sorted_slots, K, \
                                                        E, n_active, out, st);                  \
        else                                                                                    \
            launch_mode<MODE, ADT, L, TC, true, DIRECT, ONE>(W, nb, I, H, act, offsets,         \
                                                              sorted_slots, K, E, n_active, out,  \
                                                              st);                                \
        return;                                                                                 \
    }
    MOE_LPR_CASE(1) MOE_LPR_CASE(2) MOE_LPR_CASE(4) MOE_LPR_CASE(8) MOE_LPR_CASE(16)
    MOE_LPR_CASE(32) MOE_LPR_CASE(64)
#undef MOE_LPR_CASE
}

template <int ADT, int TC, bool DIRECT, bool ONE>
static void launch_both(const void* x, int H, const uint8_t* w_gate_up, const uint8_t* w_down,
                        int I, int E, int K, int n_active, const int32_t* offsets,
                        const int32_t* sorted_slots, void* h_ws, float* y_sorted, hipStream_t st) {
    launch_lpr<0, ADT, TC, DIRECT, ONE>(w_gate_up, H / 32, I, H, x, offsets, sorted_slots, K, E, n_active, h_ws,
                           st);
    launch_lpr<1, ADT, TC, DIRECT, ONE>(w_down, I / 32, I, H, h_ws, offsets, sorted_slots, K, E, n_active,
                           y_sorted, st);
}

hipError_t launch_ffn_gemv(const void* x, int x_dt, int64_t T, int H, const uint8_t* w_gate_up,
                           const uint8_t* w_down, int I, int E, int K, int N,
                           const int32_t* offsets, const int32_t* sorted_slots, void* h_ws,
                           float* y_sorted, hipStream_t st) {
    const int n_active = min(E, N);
    // One token: one chunk per expert, rows staged through LDS with coalesced
    // loads (the grid is about one wave of workgroups, so the regular stream
    // matters most).  Several tokens: direct register windows (twice the
    // workgroups per CU), one token per chunk while experts average at most one
    // slot, else two.
    auto go = [&](auto adt, auto tc, auto direct, auto one) {
        launch_both<decltype(adt)::value, decltype(tc)::value, decltype(direct)::value,
                    decltype(one)::value>(x, H, w_gate_up, w_down, I, E, K, n_active, offsets,
                                          sorted_slots, h_ws, y_sorted, st);
    };
    using F32 = std::integral_constant<int, MOE_F32>;
    using BF16 = std::integral_constant<int, MOE_BF16>;
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    using Staged = std::false_type;
    using Direct = std::true_type;
    using Single = std::true_type;
    using Many = std::false_type;
    const bool f32 = x_dt == MOE_F32;
    if (T == 1)
        f32 ? go(F32{}, One{}, Staged{}, Single{}) : go(BF16{}, One{}, Staged{}, Single{});
    else if ((int64_t)N <= E)
        f32 ? go(F32{}, One{}, Direct{}, Many{}) : go(BF16{}, One{}, Direct{}, Many{});
    else
        f32 ? go(F32{}, Two{}, Direct{}, Many{}) : go(BF16{}, Two{}, Direct{}, Many{});
    return hipGetLastError();
}

// ---- one decode layer in three launches ---------------------------------------------
// Router logits (the few-token router kernel), then gate/up with the routing
// inside, then down with the combine inside.  Each step is computed with the
// same per-token arithmetic as the four-call path (routing kernels, GEMV,
// combine), so every output is the same bit for bit; what changes is that
// top-K and the permutation run in every gate/up workgroup (no last-workgroup
// hand-off through global memory) and that no per-slot expert output y is
// stored and read back.

// Routing of a decode batch (T <= 8 tokens, T * K <= 64 slots) by one
// workgroup from the router logits: one token by wave 0 (route_one_token);
// more tokens: top-K of every token (wave w takes tokens w and w + 4), then
// the permutation of the slots by wave 0.
struct DecodeRouting {
    int32_t ids[PERM_WAVE];
    float w[PERM_WAVE];
    int32_t off[MOE_MAX_E + 1];
    int32_t ss[PERM_WAVE], sp[PERM_WAVE];
};

MOE_DEV void decode_route(const float* __restrict__ logits, int T, int E, int K, DecodeRouting& R) {
    if (T == 1) {  // one token: one wave, short dependency chains
        if (threadIdx.x < 64) route_one_token<false>(logits, E, K, R.ids, R.w, R.off, R.ss, R.sp);
        __syncthreads();
        return;
    }
    const int wave = threadIdx.x >> 6;
    const int t0 = wave, t1 = wave + 4;
    if (t1 < T) {
        float v[2][4];
        topk_load(logits + (int64_t)t0 * E, E, v[0]);
        topk_load(logits + (int64_t)t1 * E, E, v[1]);
        int32_t* const ip[2] = {R.ids + t0 * K, R.ids + t1 * K};
        float* const wp[2] = {R.w + t0 * K, R.w + t1 * K};
        topk_select_n<2>(v, E, K, ip, wp);
    } else if (t0 < T) {
        float v[4];
        topk_load(logits + (int64_t)t0 * E, E, v);
        topk_select(v, E, K, R.ids + t0 * K, R.w + t0 * K);
    }
    __syncthreads();
    if (wave == 0) permute_wave(R.ids, T * K, E, R.off, R.ss, R.sp);
    __syncthreads();
}

// Gate/up of a decode layer: every workgroup routes the batch itself (into
// LDS), then computes its tile of the by-th active expert as the expert FFN's
// gate/up kernel does, storing the hidden h by slot (token-major) instead of
// by sorted position.  Workgroup (0, 0) also stores the routing.
template <int ADT, int LPR, int TC, int UPW, bool DIRECT, bool ONE>
__global__ __launch_bounds__(256) void decode_gate_up(
    const uint8_t* __restrict__ W, int nb, int I, int H, const void* __restrict__ x,
    const float* __restrict__ logits, int T, int E, int K, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, int32_t* __restrict__ off_out, int32_t* __restrict__ ss_out,
    int32_t* __restrict__ sp_out, void* __restrict__ h_out, int wave_lds_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ DecodeRouting R;
    auto route = [&](int by, int& e, int& p0, int& n) {
        decode_route(logits, T, E, K, R);
        if (blockIdx.x == 0 && blockIdx.y == 0) {
            const int tid = threadIdx.x;
            if (tid < T * K) {
                ids_out[tid] = R.ids[tid];
                w_out[tid] = R.w[tid];
                ss_out[tid] = R.ss[tid];
                sp_out[tid] = R.sp[tid];
            }
            for (int x = tid; x <= E; x += 256) off_out[x] = R.off[x];
        }
        if (T != 1) return false;
        // one token: K distinct experts, one slot each, the by-th in sorted order
        p0 = by;
        n = 1;
        e = R.ids[R.ss[by]];
        return true;
    };
    gemv_tile<0, ADT, LPR, TC, UPW, true, DIRECT, ONE, true>(W, nb, I, H, x, R.off, R.ss, K, E,
                                                             h_out, wave_lds_bytes, smem, blockIdx.x,
                                                             blockIdx.y, route);
}

// Down and combine of a decode layer.  Workgroup (bx, t): output rows
// RR * bx .. + RR - 1 of token t.  It digitises the hidden rows of
// the token's K slots, computes those output rows of its K experts with the
// down GEMV's lane layout and arithmetic (a unit = one expert's row, LPR lanes,
// each lane a block pair in registers), and sums them in the combine's fixed
// k order with the routing weight times the expert scale, adding the
// residual for the activation-type output.  ids_t / w_t: the token's K expert
// ids and routing weights (global memory, or LDS in the one-launch decode).
// The weight windows and combine factors are loaded first; wait() then
// returns whether the hidden rows may be read (the one-launch decode waits
// there for the gate/up workgroups), and only then are they loaded.
template <int ADT, int LPR, int KB, int RR, bool COH = false, class Wait>
MOE_DEV void down_combine_tile(const uint8_t* __restrict__ Wd, int nb, int H, const void* __restrict__ hbuf,
                               const int32_t* ids_t, const float* w_t, const float* __restrict__ scale,
                               int K, const void* __restrict__ residual, int rdt,
                               float* __restrict__ out_f32, void* __restrict__ out_act, int odt,
                               uint8_t* smem, int bx, int t, Wait wait) {
    constexpr int RPS = 64 / LPR;                               // units per wave step
    constexpr int UPW = (KB * RR + 4 * RPS - 1) / (4 * RPS);  // steps per wave
    constexpr int NTB = 4;                                      // hidden quarter blocks per thread and round
    __shared__ float ys[KB][RR];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPR, q = lane % LPR;
    const int r0 = bx * RR;
    const int I = nb * 32;
    const int64_t row_bytes = (int64_t)nb * 18;
    uint32_t* dig = reinterpret_cast<uint32_t*>(smem);  // [K][16][nb] digit words
    float* dsc = reinterpret_cast<float*>(dig + K * 16 * nb);  // [K][nb] block scales

    // hidden rows -> registers, one quarter block per task (unconditional,
    // clamped loads so that their number is static); the hidden rows are
    // stored by slot, t * K + k, so their loads need no routing
    const int ntask = K * nb * 4;
    float xv[NTB][8];
    auto load_h = [&](int round) {
#pragma unroll
        for (int i = 0; i < NTB; ++i) {
            const int task = tid + 256 * (NTB * round + i);
            const bool ok = task < ntask;
            const int m = task & 3, tb = task >> 2, k = tb / nb, b = tb % nb;
            const int64_t s = (int64_t)t * K + (ok ? k : 0);
            load_quarter<ADT, COH>(hbuf, s * I + b * 32, m, xv[i]);
        }
    };
    auto digitize_h = [&](int round) {
#pragma unroll
        for (int i = 0; i < NTB; ++i) {
            const int task = tid + 256 * (NTB * round + i);
            if (task < ntask) {
                const int m = task & 3, tb = task >> 2, k = tb / nb, b = tb % nb;
                digitize_quarter(xv[i], m, dig + k * 16 * nb + b, nb, dsc + k * nb + b);
            }
        }
    };
    // this lane's weight windows: unit u = (wave * UPW + s) * RPS + g is row
    // u % RR of slot u / RR (units past the K slots load slot K-1's); each lane
    // reads the expert of its own slot (a few distinct addresses per wave)
    const int qq = min(q, nb / 2 - 1);
    uint32_t wd[UPW][9];
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
        const int u = (wave * UPW + s) * RPS + g;
        const int k = min(u / RR, K - 1), r = u % RR;
        const uint8_t* pw = Wd + ((int64_t)ids_t[k] * H + r0 + r) * row_bytes + 36 * qq;
        const u32x4a4 a = *reinterpret_cast<const u32x4a4*>(pw);
        const u32x4a4 b = *reinterpret_cast<const u32x4a4*>(pw + 16);
        const uint32_t c = *reinterpret_cast<const uint32_t*>(pw + 32);
        wd[s][0] = a.x; wd[s][1] = a.y; wd[s][2] = a.z; wd[s][3] = a.w;
        wd[s][4] = b.x; wd[s][5] = b.y; wd[s][6] = b.z; wd[s][7] = b.w;
        wd[s][8] = c;
    }
    // combine factors (used last)
    float ck[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int kk = min(k, K - 1);
        ck[k] = w_t[kk] * (scale ? scale[ids_t[kk]] : 1.f);
    }
    if (!wait()) return;
    load_h(0);
    digitize_h(0);
    const int rounds = (ntask + 256 * NTB - 1) / (256 * NTB);
    for (int round = 1; round < rounds; ++round) {
        load_h(round);
        digitize_h(round);
    }
    __syncthreads();  // the digits of all K slots are in LDS
    const int nblk_here = min(2, max(0, nb - 2 * q));
    const int qp = min(q, nb / 2 - 1);
#pragma unroll
    for (int s = 0; s < UPW; ++s) {
        const int u = (wave * UPW + s) * RPS + g;
        const int k = u / RR, r = u % RR;
        const bool valid = k < K;
        const int kk = min(k, K - 1);
        const PairDec w = reg_pair(wd[s], valid ? nblk_here : 0);
        uint32_t xa[16], xb[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint2 v = reinterpret_cast<const uint2*>(dig + (kk * 16 + i) * nb)[qp];
            xa[i] = v.x;
            xb[i] = v.y;
        }
        const float2 sv = reinterpret_cast<const float2*>(dsc + kk * nb)[qp];
        const float y = group_sum<LPR>(pair_acc(w, xa, xb, sv.x, sv.y));
        if (valid && q == LPR - 1) ys[k][r] = y;
    }
    __syncthreads();
    if (tid < RR) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < KB; ++k)
            if (k < K) acc = fmaf(ck[k], ys[k][tid], acc);
        const int64_t o = (int64_t)t * H + r0 + tid;
        if (out_f32) out_f32[o] = acc;
        if (out_act) store_act(out_act, odt, o, residual ? acc + load_act(residual, rdt, o) : acc);
    }
}

template <int ADT, int LPR, int KB, int RR>
__global__ __launch_bounds__(256) void decode_down_combine(
    const uint8_t* __restrict__ Wd, int nb, int H, const void* __restrict__ hbuf,
    const int32_t* __restrict__ ids, const float* __restrict__ tw,
    const float* __restrict__ scale, int K,
    const void* __restrict__ residual, int rdt, float* __restrict__ out_f32,
    void* __restrict__ out_act, int odt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int t = blockIdx.y;
    down_combine_tile<ADT, LPR, KB, RR>(Wd, nb, H, hbuf, ids + (int64_t)t * K, tw + (int64_t)t * K, scale,
                                        K, residual, rdt, out_f32, out_act, odt, smem, blockIdx.x, t,
                                        [] { return true; });
}

// ---- one-token decode: gate/up and down in one launch ------------------------------
// Workgroups 0 .. ng-1 are the gate/up tiles of decode_gate_up (bx = b % wgs,
// by = b / wgs); workgroups ng .. ng+nd-1 the down + combine tiles of
// decode_down_combine (output rows RR * (b - ng) ..).  A down workgroup routes
// the token itself (the same selection as every gate/up workgroup), loads its
// weight windows and combine factors, and only then waits until every gate/up
// workgroup has stored its part of h.
//
// Hand-over without cache maintenance: h is stored with agent-scope relaxed
// atomic stores and read with agent-scope relaxed atomic loads, both coherent
// across the XCDs' L2 caches, so neither side needs an L2 write-back or
// invalidate (each costs microseconds when hundreds of workgroups issue one).
// A gate/up workgroup waits until its stores are acknowledged (vmcnt 0),
// crosses a barrier and bumps counter b mod DECODE_CTR_LINES; the counters sit
// on separate 256-byte lines, since hundreds of increments and polls on one
// address serialise at its memory channel.  Wave 0 of a down workgroup polls
// all counters (one per lane) until each has its share of ng.
//
// The down workgroups carry the highest block numbers and workgroups are
// dispatched in order, so every gate/up workgroup is resident or finished
// before any down workgroup waits; the wait is bounded all the same
// (DECODE_WAIT_LIMIT polls, each a memory round trip and a short sleep: about
// a second): on expiry the timeout flag (ctr[1]) is set and the workgroup
// stores nothing.  The counters are zeroed by the router launch of the same
// call.  Outputs equal the two-launch path's bit for bit.
constexpr int DECODE_WAIT_LIMIT = 1 << 20;
static_assert(DECODE_CTR_LINES <= 64, "one lane of wave 0 watches each counter");

template <int ADT, int LPR, int UPW, int LPRD, int KB, int RR>
__global__ __launch_bounds__(256) void decode_ffn_one(
    const uint8_t* __restrict__ W, const uint8_t* __restrict__ Wd, int nb, int nbd, int I, int H,
    const void* __restrict__ x, const float* __restrict__ logits, int E, int K,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* __restrict__ off_out,
    int32_t* __restrict__ ss_out, int32_t* __restrict__ sp_out, void* __restrict__ h,
    int wave_lds_bytes, int wgs, int ng, int* __restrict__ ctr, const float* __restrict__ scale,
    const void* __restrict__ residual, int rdt, float* __restrict__ out_f32,
    void* __restrict__ out_act, int odt) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ DecodeRouting R;
    __shared__ int s_ok;
    const int b = blockIdx.x;
    if (b < ng) {
        const int bx = b % wgs, by = b / wgs;
        auto route = [&](int, int& e, int& p0, int& n) {
            decode_route(logits, 1, E, K, R);
            if (b == 0) {
                const int tid = threadIdx.x;
                if (tid < K) {
                    ids_out[tid] = R.ids[tid];
                    w_out[tid] = R.w[tid];
                    ss_out[tid] = R.ss[tid];
                    sp_out[tid] = R.sp[tid];
                }
                for (int xx = tid; xx <= E; xx += 256) off_out[xx] = R.off[xx];
            }
            // K distinct experts, one slot each, the by-th in sorted order
            p0 = by;
            n = 1;
            e = R.ids[R.ss[by]];
            return true;
        };
        gemv_tile<0, ADT, LPR, 1, UPW, true, false, true, true, true>(
            W, nb, I, H, x, R.off, R.ss, K, E, h, wave_lds_bytes, smem, bx, by, route);
        // the agent-scope stores of h are complete (acknowledged) before the
        // barrier, so the increment after it publishes them without an L2
        // write-back
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(ctr + DECODE_CTR_STRIDE * (b % DECODE_CTR_LINES), 1,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    decode_route(logits, 1, E, K, R);
    auto wait = [&]() {
        if (threadIdx.x < 64) {
            // lane j < DECODE_CTR_LINES watches counter j, which gate/up
            // workgroups b = j mod DECODE_CTR_LINES bump
            const int j = threadIdx.x;
            const int need = j < DECODE_CTR_LINES
                                 ? ng / DECODE_CTR_LINES + (j < ng % DECODE_CTR_LINES ? 1 : 0)
                                 : 0;
            int* cj = ctr + DECODE_CTR_STRIDE * min(j, DECODE_CTR_LINES - 1);
            int it = 0;
            while (__ballot(j < DECODE_CTR_LINES &&
                            __hip_atomic_load(cj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) &&
                   it < DECODE_WAIT_LIMIT) {
                __builtin_amdgcn_s_sleep(1);
                ++it;
            }
            if (j == 0) {
                s_ok = it < DECODE_WAIT_LIMIT;
                if (!s_ok) __hip_atomic_store(ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
        return s_ok != 0;
    };
    down_combine_tile<ADT, LPRD, KB, RR, true>(Wd, nbd, H, h, R.ids, R.w, scale, K, residual, rdt, out_f32,
                                         out_act, odt, smem, b - ng, 0, wait);
}

// output rows per workgroup of the fused down + combine (a divisor of 64)
constexpr int DECODE_DOWN_ROWS = 16;

size_t decode_down_lds_bytes(int K, int I) { return (size_t)K * (I / 32) * 17 * sizeof(uint32_t); }

bool decode_layer_supported(int64_t T, int H, int I, int K) {
    return T >= 1 && T <= ROUTER_GEMV_MAX_T && T * K <= PERM_WAVE && H % 64 == 0 && I % 64 == 0 &&
           decode_down_lds_bytes(K, I) <= 64 * 1024;
}

template <int ADT, int LPR, int TC, bool DIRECT, bool ONE>
static void launch_decode_gate_up(const uint8_t* W, int nb, int I, int H, const void* x,
                                  const float* logits, int T, int E, int K, int n_active,
                                  int32_t* ids, float* w, int32_t* off, int32_t* ss, int32_t* sp,
                                  void* h, hipStream_t st) {
    constexpr int RPS = 64 / LPR;
    constexpr int UPW = steps_per_wave<0, LPR, DIRECT>();
    constexpr int RPW = RPS * UPW;
    const int wgs = (I + 4 * RPW - 1) / (4 * RPW);
    constexpr int NCH = (RPW * 36 * LPR + 15 + 1023) / 1024;
    const int wave_lds = DIRECT ? 0 : 2 * NCH * 1024;
    const size_t lds = (size_t)4 * wave_lds + (size_t)TC * nb * 17 * sizeof(uint32_t);
    decode_gate_up<ADT, LPR, TC, UPW, DIRECT, ONE><<<dim3(wgs, n_active), 256, lds, st>>>(
        W, nb, I, H, x, logits, T, E, K, ids, w, off, ss, sp, h, wave_lds);
}

hipError_t launch_decode_layer(const void* x, int x_dt, int T, int H, const float* logits, int E,
                               int K, const uint8_t* w_gate_up, const uint8_t* w_down, int I,
                               const float* scale, int32_t* ids, float* w, int32_t* off,
                               int32_t* ss, int32_t* sp, const void* residual, int rdt,
                               float* out_f32, void* out_act, int odt, void* h_ws, int* ctr,
                               hipStream_t st) {
    const int N = T * K, n_active = min(E, N);
    // one token, gate/up rows of 33..64 block pairs (LPR 64), down rows of 9..16
    // (LPR 16), at most 8 experts: gate/up and down in one launch
    if (T == 1 && K <= 8 && ctr && H / 64 > 32 && H / 64 <= 64 && I / 64 > 8 && I / 64 <= 16) {
        constexpr int LPR = 64, LPRD = 16, KB = 8, RR = DECODE_DOWN_ROWS;
        constexpr int UPW = steps_per_wave<0, LPR, false>();
        constexpr int RPW = (64 / LPR) * UPW;
        constexpr int NCH = (RPW * 36 * LPR + 15 + 1023) / 1024;
        const int nb = H / 32, nbd = I / 32;
        const int wgs = (I + 4 * RPW - 1) / (4 * RPW), ng = wgs * n_active, nd = H / RR;
        const int wave_lds = 2 * NCH * 1024;
        const size_t lds = std::max((size_t)4 * wave_lds + (size_t)nb * 17 * sizeof(uint32_t),
                                    decode_down_lds_bytes(K, I));
        auto go = [&](auto adt) {
            constexpr int A = decltype(adt)::value;
            decode_ffn_one<A, LPR, UPW, LPRD, KB, RR><<<ng + nd, 256, lds, st>>>(
                w_gate_up, w_down, nb, nbd, I, H, x, logits, E, K, ids, w, off, ss, sp, h_ws, wave_lds,
                wgs, ng, ctr, scale, residual, rdt, out_f32, out_act, odt);
        };
        if (x_dt == MOE_F32)
            go(std::integral_constant<int, MOE_F32>{});
        else
            go(std::integral_constant<int, MOE_BF16>{});
        return hipGetLastError();
    }
    // gate/up: the expert FFN's choice of chunk size and load path
    auto gu = [&](auto adt, auto tc, auto direct, auto one) {
        constexpr int A = decltype(adt)::value, TC = decltype(tc)::value;
        constexpr bool D = decltype(direct)::value, O = decltype(one)::value;
        const int nb = H / 32, pairs = nb / 2;
#define MOE_DGU_CASE(L)                                                                        \
        if (pairs <= L) {                                                                      \
            launch_decode_gate_up<A, L, TC, D, O>(w_gate_up, nb, I, H, x, logits, T, E, K,     \
                                                  n_active, ids, w, off, ss, sp, h_ws, st);    \
            return;                                                                            \
        }
        MOE_DGU_CASE(1) MOE_DGU_CASE(2) MOE_DGU_CASE(4) MOE_DGU_CASE(8) MOE_DGU_CASE(16)
        MOE_DGU_CASE(32) MOE_DGU_CASE(64)
#undef MOE_DGU_CASE
    };
    using F32 = std::integral_constant<int, MOE_F32>;
    using BF16 = std::integral_constant<int, MOE_BF16>;
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    const bool f32 = x_dt == MOE_F32;
    if (T == 1)
        f32 ? gu(F32{}, One{}, std::false_type{}, std::true_type{})
            : gu(BF16{}, One{}, std::false_type{}, std::true_type{});
    else if (N <= E)
        f32 ? gu(F32{}, One{}, std::true_type{}, std::false_type{})
            : gu(BF16{}, One{}, std::true_type{}, std::false_type{});
    else
        f32 ? gu(F32{}, Two{}, std::true_type{}, std::false_type{})
            : gu(BF16{}, Two{}, std::true_type{}, std::false_type{});
    // down + combine
    const int nb = I / 32, pairs = nb / 2;
    const size_t lds = decode_down_lds_bytes(K, I);
    constexpr int RR = DECODE_DOWN_ROWS;
    const dim3 grid(H / RR, T);
    auto dc = [&](auto adt, auto kb) {
        constexpr int A = decltype(adt)::value, KB = decltype(kb)::value;
#define MOE_DDC_CASE(L)                                                                          \
        if (pairs <= L) {                                                                        \
            decode_down_combine<A, L, KB, RR><<<grid, 256, lds, st>>>(                           \
                w_down, nb, H, h_ws, ids, w, scale, K, residual, rdt, out_f32, out_act, odt);     \
            return;                                                                              \
        }
        MOE_DDC_CASE(1) MOE_DDC_CASE(2) MOE_DDC_CASE(4) MOE_DDC_CASE(8) MOE_DDC_CASE(16)
        MOE_DDC_CASE(32) MOE_DDC_CASE(64)
#undef MOE_DDC_CASE
    };
    using K8 = std::integral_constant<int, 8>;
    using K16 = std::integral_constant<int, 16>;
    if (K <= 8)
        f32 ? dc(F32{}, K8{}) : dc(BF16{}, K8{});
    else
        f32 ? dc(F32{}, K16{}) : dc(BF16{}, K16{});
    return hipGetLastError();
}

// ---- plain Q4_0 linear layer: y [T, R] = x [T, H] W^T --------------------------
// The down-product kernels with one expert holding every token in order
// (offsets {0, T}, slots 0..T-1, written by dense_index).
__global__ void dense_index(int64_t T, int32_t* __restrict__ offsets, int32_t* __restrict__ slots) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < T) slots[i] = (int32_t)i;
    if (i == 0) {
        offsets[0] = 0;
        offsets[1] = (int32_t)T;
    }
}

hipError_t launch_dense_index(int64_t T, int32_t* offsets, int32_t* slots, hipStream_t st) {
    dense_index<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(T, offsets, slots);
    return hipGetLastError();
}

hipError_t launch_linear_gemv(const void* x, int x_dt, int64_t T, int H, const uint8_t* W, int R,
                              const int32_t* offsets, const int32_t* slots, float* y,
                              hipStream_t st) {
    auto go = [&](auto adt, auto tc, auto direct) {
        launch_lpr<1, decltype(adt)::value, decltype(tc)::value, decltype(direct)::value, false>(
            W, H / 32, H, R, x, offsets, slots, 1, 1, 1, y, st);
    };
    using F32 = std::integral_constant<int, MOE_F32>;
    using BF16 = std::integral_constant<int, MOE_BF16>;
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    const bool f32 = x_dt == MOE_F32;
    if (T == 1)
        f32 ? go(F32{}, One{}, std::false_type{}) : go(BF16{}, One{}, std::false_type{});
    else
        f32 ? go(F32{}, Two{}, std::true_type{}) : go(BF16{}, Two{}, std::true_type{});
    return hipGetLastError();
}

}  // namespace moe
