// Expert FFN for many tokens per expert (prefill): grouped GEMM on bf16 MFMA,
// gfx950.
//
// The slots routed to one expert form a dense product with that expert's Q4_0
// matrix, which is read in place.  One K step of v_mfma_f32_16x16x32_bf16 is
// exactly one Q4_0 block, so the block scale can be applied to the MFMA result
// before it joins the running sum, and no dequantised weight is ever rounded:
//
//   * the nibbles q enter the MFMA as the bf16 values 1 + q/16, which are exact
//     (the nibble ORed into bits 3..6 of the mantissa of 1.0: two bit
//     operations per pair of values, no float arithmetic);
//   * the accumulator input is C = -1.5 * (sum of the block's 32 activations),
//     so the MFMA returns sum x (1 + q/16) - 1.5 sum x = sum x (q - 8) / 16,
//     exact products with fp32 accumulation;
//   * the fp16 block scale d then multiplies that partial in fp32,
//     acc += d * tmp, and the result is 16 * acc.
//
// Within a block, the MFMA's k order is chosen to make the nibble unpacking
// cheap (lane group g takes qs bytes 4g..4g+3, both nibbles); the activations
// are stored in the same order.  A prep kernel writes the activations in that
// order together with the block sums; the gate/up epilogue writes the hidden h
// (rounded to bf16) the same way, so the down product reads it directly.
//
// Tiles: 128 slots x 128 weight rows per workgroup of 4 waves (2 x 2, 64 x 64
// per wave = 4 x 4 MFMA tiles); two Q4_0 blocks per LDS stage.  For gate/up a
// tile's 128 rows are 64 gate rows and the 64 up rows of the same hidden
// columns, and each wave holds gate and up of the same (slot, column) in
// matching registers, so GELU(g) * u is formed in the epilogue.
#include "kernels.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MT = 128;        // slots per tile
constexpr int NT = 128;        // weight rows per tile
constexpr int ROWB = 80;       // LDS bytes per (row, block): 64 data + 16 pad (no bank conflicts)
// one LDS slot: A [MT rows][80 B], B [NT rows][80 B], D [NT] scales, C [MT] sums
constexpr int SLOT_BYTES = MT * ROWB + NT * ROWB + 4 * (NT + MT);
constexpr int LDS_BYTES = 3 * SLOT_BYTES;

// Position, inside a 32-element block as the MFMA reads it, of element j.
// Lane group g holds k slots 8g..8g+7 = elements 4g, 4g+2, 4g+16, 4g+18,
// 4g+1, 4g+3, 4g+17, 4g+19 (see dq_group).
MOE_DEV int perm_pos(int j) {
    const int hi = j >> 4, g = (j & 15) >> 2, r = j & 3;
    return 8 * g + ((r & 1) << 2) + (r >> 1) + (hi << 1);
}

// One qs dword (bytes 4g..4g+3 of a block: nibbles n0..n7 from bit 0 up, n0 =
// element 4g, n1 = element 4g+16, n2 = element 4g+1, ...) -> four bf16 pairs
// holding 1 + q/16 for (n0,n4), (n1,n5), (n2,n6), (n3,n7).
MOE_DEV u32x4 dq_group(uint32_t w) {
    const uint32_t M = 0x00780078u, ONE = 0x3F803F80u;
    u32x4 r;
    r.x = ((w << 3) & M) | ONE;
    r.y = ((w >> 1) & M) | ONE;
    r.z = ((w >> 5) & M) | ONE;
    r.w = ((w >> 9) & M) | ONE;
    return r;
}

MOE_DEV f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Tile lookup: tiles are numbered expert by expert, ceil(count/MT) per expert.
// Wave 0 scans the expert counts (up to 4 experts per lane); returns false for
// a tile number past the last tile.
__device__ bool find_tile(const int32_t* __restrict__ offsets, int E, int tile, int* s_res,
                          int& e_out, int& base, int& cnt) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int c[4], t[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane * 4 + q;
            c[q] = e < E ? offsets[e + 1] - offsets[e] : 0;
            t[q] = (c[q] + MT - 1) / MT;
            tot += t[q];
        }
        int incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        int run = incl - tot;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (tile >= run && tile < run + t[q]) {
                const int e = lane * 4 + q, k = tile - run;
                s_res[0] = e;
                s_res[1] = offsets[e] + k * MT;
                s_res[2] = min(MT, c[q] - k * MT);
            }
            run += t[q];
        }
        if (lane == 63 && tile >= incl) s_res[0] = -1;
    }
    __syncthreads();
    e_out = s_res[0];
    base = s_res[1];
    cnt = s_res[2];
    return e_out >= 0;
}

// MODE 0: gate/up.  act = permuted x [T][H], csum = -1.5 * block sums [T][H/32],
//         W = w_gate_up, rows_e = 2I, ncols = I; writes h (permuted) and its
//         block sums.
// MODE 1: down.     act = permuted h [N][I], csum [N][I/32], W = w_down,
//         rows_e = ncols = H; writes y_sorted.
//
// Pipeline over the K blocks (one Q4_0 block per stage, three LDS slots and
// three register sets): iteration j stores stage j+1 into LDS, issues the
// global loads of stage j+3, runs the MFMAs of stage j, and ends on a barrier.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_mfma(
    const uint16_t* __restrict__ act, const float* __restrict__ csum, const uint8_t* __restrict__ W,
    int nb, int rows_e, int ncols, int n_tiles, int tiles_per_xcd, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, int K, int E, uint16_t* __restrict__ h_out,
    float* __restrict__ hsum_out, float* __restrict__ y_out) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_res[3];

    // XCD-aware numbering: consecutive tile numbers (the column tiles of one
    // slot tile, then the next slot tile of the same expert) share an XCD's L2.
    const int bid = blockIdx.x;
    const int lin = (bid & 7) * tiles_per_xcd + (bid >> 3);
    const int mtile = lin / n_tiles, ntile = lin - mtile * n_tiles;
    int e, base, cnt;
    if (!find_tile(offsets, E, mtile, s_res, e, base, cnt)) return;
    e = __builtin_amdgcn_readfirstlane(e);
    base = __builtin_amdgcn_readfirstlane(base);
    cnt = __builtin_amdgcn_readfirstlane(cnt);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const size_t rowbytes = (size_t)nb * 18;
    const int col0 = ntile * (MODE == 0 ? NT / 2 : NT);  // first hidden column / output row

    // ---- staging role: tile rows r4 and r4 + 64, 16-byte chunk / qs dword q4 ----
    const int r4 = tid >> 2, q4 = tid & 3;
    const uint16_t* a_src[2];
    const float* c_src[2];
    size_t w_off[2];  // byte offset of the weight row in W (W is 16-byte aligned)
    int sslot[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = r4 + 64 * h;
        const int p = base + min(r, cnt - 1);
        const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
        a_src[h] = act + arow * (int64_t)nb * 32 + 8 * q4;
        c_src[h] = csum + arow * (int64_t)nb;
        int wrow;
        if (MODE == 0) {  // tile rows 0..63 gate, 64..127 up, of hidden columns col0 + (0..63)
            wrow = min(col0 + r4, ncols - 1) + h * ncols;
            sslot[h] = (r4 >> 5) * 64 + (((r4 >> 4) & 1) + 2 * h) * 16 + (r4 & 15);
        } else {
            wrow = min(col0 + r, rows_e - 1);
            sslot[h] = r;
        }
        w_off[h] = ((size_t)e * rows_e + wrow) * rowbytes;
    }

    // ---- per-wave extent (uniform) ----
    const int m_rows = cnt - wm * 64;
    const int mfa = m_rows <= 0 ? 0 : min(4, (m_rows + 15) >> 4);
    int nfa;
    if (MODE == 0)
        nfa = (col0 + wn * 32 < ncols) ? 4 : 0;
    else
        nfa = max(0, min(4, (ncols - (col0 + wn * 64)) >> 4));
    const bool active = mfa > 0 && nfa > 0;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // register stage: 2 activation chunks, 2 qs dword pairs, 2 scales, 2 sums
    struct Stage {
        u32x4a4 a[2];
        uint32_t lo[2], hi[2];
        uint32_t d[2];
        float c[2];
        int sh[2];
    };
    auto load = [&](Stage& S, int b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            S.a[h] = *(const u32x4a4*)(a_src[h] + (int64_t)b * 32);
            const size_t bo = w_off[h] + (size_t)b * 18;         // block start
            const size_t qo = bo + 2 + 4 * q4;                       // this lane's qs dword
            const uint32_t* qw = (const uint32_t*)(W + (qo & ~(size_t)3));
            S.sh[h] = (int)(qo & 3);
            S.lo[h] = qw[0];
            // branch-free (every lane issues the same loads, which keeps the
            // wait counts exact): a straddling qs dword takes its last two bytes
            // from a 16-bit load that ends inside the block; otherwise the
            // 16-bit load rereads the first dword and is ignored
            S.hi[h] = (uint32_t)*(const uint16_t*)(qw + (S.sh[h] ? 1 : 0));
            S.d[h] = (uint32_t)*(const uint16_t*)(W + bo);
            S.c[h] = c_src[h][b];
        }
    };
    auto store = [&](const Stage& S, int slot) {
        uint8_t* A_lds = smem + slot * SLOT_BYTES;
        uint8_t* B_lds = A_lds + MT * ROWB;
        float* D_lds = (float*)(B_lds + NT * ROWB);
        float* C_lds = D_lds + NT;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = r4 + 64 * h;
            *(u32x4*)(A_lds + r * ROWB + 16 * q4) = (u32x4){S.a[h].x, S.a[h].y, S.a[h].z, S.a[h].w};
            const uint32_t w = __builtin_amdgcn_alignbyte(S.hi[h], S.lo[h], S.sh[h]);
            *(u32x4*)(B_lds + sslot[h] * ROWB + 16 * q4) = dq_group(w);
            if (q4 == 0) {
                C_lds[r] = S.c[h];
                const int s = sslot[h];
                D_lds[(((s >> 6) * 16) + (s & 15)) * 4 + ((s >> 4) & 3)] = f16_bits_to_f32(S.d[h]);
            }
        }
    };
    auto compute = [&](int slot) {
        const uint8_t* A_lds = smem + slot * SLOT_BYTES;
        const uint8_t* B_lds = A_lds + MT * ROWB;
        const float* D_lds = (const float*)(B_lds + NT * ROWB);
        const float* C_lds = D_lds + NT;
        const f32x4 dv = *(const f32x4*)&D_lds[(wn * 16 + l16) * 4];
        u32x4 bq[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
            bq[nf] = *(const u32x4*)(B_lds + (wn * 64 + nf * 16 + l16) * ROWB + 16 * g);
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
            const int r = wm * 64 + mf * 16;
            const u32x4 a = *(const u32x4*)(A_lds + (r + l16) * ROWB + 16 * g);
            const f32x4 c = *(const f32x4*)&C_lds[r + 4 * g];
            f32x4 t[4];
#pragma unroll
            for (int nf = 0; nf < 4; ++nf) t[nf] = mfma_bf16(a, bq[nf], c);
#pragma unroll
            for (int nf = 0; nf < 4; ++nf)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mf][nf][i] = fmaf(dv[nf], t[nf][i], acc[mf][nf][i]);
        }
    };

    // stage s lives in register set s % 3 and LDS slot s % 3: its loads are
    // issued two iterations before the iteration that stores it to LDS
    Stage R0, R1, R2;
    load(R0, 0);
    load(R1, min(1, nb - 1));
    load(R2, min(2, nb - 1));
    store(R0, 0);
    lds_barrier();
    auto iter = [&](int jj, int cs, int ns, const Stage& Rst, Stage& Rld) {
        if (jj + 1 < nb) store(Rst, ns);
        // unconditional (clamped past the end) so every path issues the same
        // loads and the compiler's wait counts stay exact
        load(Rld, min(jj + 3, nb - 1));
        if (active) compute(cs);
        lds_barrier();
    };
    for (int j = 0; j < nb; j += 3) {
        iter(j, 0, 1, R1, R0);
        if (j + 1 >= nb) break;
        iter(j + 1, 1, 2, R2, R1);
        if (j + 2 >= nb) break;
        iter(j + 2, 2, 0, R0, R2);
    }

    if (!active) return;
    if (MODE == 0) {
        // h = GELU(g) * u for hidden columns col0 + wn*32 + (0..31): one Q4_0
        // block of the down product's K, written in the MFMA order with its sum.
        const int I = ncols, nbh = I >> 5;
        const int hblk = (col0 >> 5) + wn;
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
            if (mf < mfa) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 64 + mf * 16 + 4 * g + i;
                    const bool ok = r < cnt;
                    const int64_t p = base + min(r, cnt - 1);
                    float s = 0.f;
#pragma unroll
                    for (int f = 0; f < 2; ++f) {
                        const float gv = 16.f * acc[mf][f][i], uv = 16.f * acc[mf][2 + f][i];
                        const uint16_t hb = f32_to_bf16(gelu_tanh(gv) * uv);
                        s += bf16_to_f32(hb);
                        if (ok) h_out[p * I + hblk * 32 + perm_pos(f * 16 + l16)] = hb;
                    }
                    // sum over the 16 lanes holding this row's columns
                    s += dpp_f32<DPP_QUAD_XOR1>(0.f, s);
                    s += dpp_f32<DPP_QUAD_XOR2>(0.f, s);
                    s += dpp_f32<DPP_ROW_HALF_MIRROR>(0.f, s);
                    s += dpp_f32<DPP_ROW_MIRROR>(0.f, s);
                    if (ok && l16 == 0) hsum_out[p * nbh + hblk] = -1.5f * s;
                }
            }
        }
    } else {
        const int H = ncols;
#pragma unroll
        for (int mf = 0; mf < 4; ++mf) {
            if (mf < mfa) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wm * 64 + mf * 16 + 4 * g + i;
                    if (r < cnt) {
                        float* yp = y_out + (int64_t)(base + r) * H + col0 + wn * 64 + l16;
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf)
                            if (nf < nfa) yp[nf * 16] = 16.f * acc[mf][nf][i];
                    }
                }
            }
        }
    }
}

// Activations -> MFMA block order, plus -1.5 * block sums.  One thread per
// (token, block).
__global__ __launch_bounds__(256) void ffn_mfma_prep(const uint16_t* __restrict__ x, int64_t nblocks,
                                                     uint16_t* __restrict__ xp,
                                                     float* __restrict__ xs) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nblocks) return;
    const u32x4* src = (const u32x4*)(x + i * 32);
    uint32_t v[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 t = src[c];
        v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
    }
    uint16_t e[32], o[32];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        e[j] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
        s += bf16_to_f32(e[j]);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) o[perm_pos(j)] = e[j];
    u32x4* dst = (u32x4*)(xp + i * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u32x4 t;
        t.x = o[8 * c] | ((uint32_t)o[8 * c + 1] << 16);
        t.y = o[8 * c + 2] | ((uint32_t)o[8 * c + 3] << 16);
        t.z = o[8 * c + 4] | ((uint32_t)o[8 * c + 5] << 16);
        t.w = o[8 * c + 6] | ((uint32_t)o[8 * c + 7] << 16);
        dst[c] = t;
    }
    xs[i] = -1.5f * s;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t ffn_mfma_ws_bytes(int64_t T, int H, int I, int64_t N) {
    return align256((size_t)T * H * 2) + align256((size_t)T * (H / 32) * 4) +
           align256((size_t)N * I * 2) + align256((size_t)N * (I / 32) * 4);
}

hipError_t launch_ffn_mfma(const void* x, int64_t T, int H, const uint8_t* w_gate_up,
                           const uint8_t* w_down, int I, int E, int K, int N,
                           const int32_t* offsets, const int32_t* sorted_slots, void* ws,
                           float* y_sorted, hipStream_t st) {
    uint8_t* p = (uint8_t*)ws;
    uint16_t* xp = (uint16_t*)p;
    p += align256((size_t)T * H * 2);
    float* xs = (float*)p;
    p += align256((size_t)T * (H / 32) * 4);
    uint16_t* hp = (uint16_t*)p;
    p += align256((size_t)N * I * 2);
    float* hs = (float*)p;

    const int64_t nblk = T * (H / 32);
    ffn_mfma_prep<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>((const uint16_t*)x, nblk, xp, xs);

    // slot tiles: sum over experts of ceil(count / MT) <= N / MT + (experts hit)
    const int mtiles = N / MT + min(E, N);
    {
        const int n_tiles = (I + NT / 2 - 1) / (NT / 2);
        const int total = (mtiles * n_tiles + 7) / 8 * 8;
        ffn_mfma<0><<<total, 256, LDS_BYTES, st>>>(xp, xs, w_gate_up, H / 32, 2 * I, I, n_tiles,
                                                   total / 8, offsets, sorted_slots, K, E, hp, hs,
                                                   nullptr);
    }
    {
        const int n_tiles = (H + NT - 1) / NT;
        const int total = (mtiles * n_tiles + 7) / 8 * 8;
        ffn_mfma<1><<<total, 256, LDS_BYTES, st>>>(hp, hs, w_down, I / 32, H, H, n_tiles, total / 8,
                                                   offsets, sorted_slots, K, E, nullptr, nullptr,
                                                   y_sorted);
    }
    return hipGetLastError();
}

}  // namespace moe
