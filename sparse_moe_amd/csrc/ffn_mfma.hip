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
// Tiles: 128 slots x 256 weight rows per workgroup of 4 waves, each wave 128
// slots x 64 rows (8 x 4 MFMA tiles); an expert's last tile may take up to 160
// slots (10 x 4); two Q4_0 blocks per stage.  For gate/up
// a wave's 64 rows are 32 gate rows and the 32 up rows of the same hidden
// columns, so each lane holds gate and up of the same (slot, column) in
// matching registers and GELU(g) * u is formed in the epilogue.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MT = 128;        // slots per tile
// In the XCD-run numbering an expert's last tile takes up to MTX slots (10
// fragments of 16) instead of leaving a tile of at most 32 slots behind.
constexpr int MTX = 160;
constexpr int NT = 256;        // weight rows per tile (64 per wave)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt for vector memory only: vmcnt <= n (expcnt and lgkmcnt left alone)
template <int N>
MOE_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the direct-load pipeline: waits for this wave's LDS
// reads and writes (lgkmcnt) but not for its direct loads in flight, which a
// memory-model fence would drain; the empty asm statements keep the compiler
// from moving LDS accesses across it.  Completion of the direct loads a stage
// needs is waited for explicitly (wait_vmcnt) before the barrier.
MOE_DEV void stage_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt(63) and expcnt(7): no wait
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct loads into LDS written out as instructions (16 or 4 bytes per lane;
// lane i's bytes land at LDS address lds + size * i; M0 holds the address, with
// the one wait state after writing it that the hardware needs).  Issued this
// way they are invisible to the compiler's wait insertion, which tracks direct
// loads per LDS array in a handful of slots and, past those or across the
// ring's loop, waited for every load in flight before the reads of a stage;
// the kernel waits for them itself (wait_vmcnt before each stage barrier).
// They have no register results, so nothing the compiler allocates can be
// overwritten by a load in flight.
typedef int i32x4 __attribute__((ext_vector_type(4)));
// buffer resource for raw, unbounded 32-bit offsets from a base address (the
// fourth word selects 32-bit data, as untyped loads need)
MOE_DEV i32x4 buffer_rsrc(const void* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return (i32x4){(int)__builtin_amdgcn_readfirstlane((uint32_t)a),
                   (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu), -1, 0x00020000};
}
MOE_DEV void dma16(const void* lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds)), "v"(voff), "s"(rsrc),
                    "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}
MOE_DEV void dma4(const void* lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds)), "v"(voff), "s"(rsrc),
                    "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}

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
MOE_DEV u32x4 dq_group(uint32_t w, uint32_t M) {
    const uint32_t ONE = 0x3F803F80u;
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

// One stage (a pair of Q4_0 blocks) of a wave's products: NF 16-row weight
// fragments (48-byte rows from WL) against MF 16-slot fragments of the staged
// activations Sa [2][AROWS][64 B] with their sums Sc [2][AROWS], added into acc.
template <int MF, int NF, int AROWS>
MOE_DEV void stage_products(const uint8_t* __restrict__ Sa, const float* __restrict__ Sc,
                            const uint8_t* __restrict__ WL, int g, int l16, int swz, int q1off,
                            uint32_t nib_mask, f32x4 (&acc)[MF][NF]) {
    // The weight words of both blocks are read first, so the LDS round
    // trips of block 1 pass under block 0's MFMAs (read per block, each
    // block began with four dependent reads in turn).  Block 0: the scale
    // and bytes 2 + 4g .. 5 + 4g of the pair (two dwords and an
    // alignbyte); block 1: the scale and bytes 20 + 4g .. 23 + 4g.
    uint32_t w0lo[NF], w0hi[NF], w1q[NF], d0b[NF], d1b[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
        const uint8_t* rp = WL + nf * 16 * 48;
        w0lo[nf] = *(const uint32_t*)(rp + 4 * g);
        w0hi[nf] = *(const uint32_t*)(rp + 4 * g + 4);
        d0b[nf] = *(const uint16_t*)rp;
    }
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
        const uint8_t* rp = WL + nf * 16 * 48;
        w1q[nf] = *(const uint32_t*)(rp + q1off);
        d1b[nf] = *(const uint16_t*)(rp + 18);
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        float dv[NF];
        u32x4 bq[NF];
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
            if (blk == 0) {
                dv[nf] = f16_bits_to_f32((uint16_t)d0b[nf]);
                bq[nf] = dq_group(__builtin_amdgcn_alignbyte(w0hi[nf], w0lo[nf], 2), nib_mask);
            } else {
                dv[nf] = f16_bits_to_f32((uint16_t)d1b[nf]);
                bq[nf] = dq_group(w1q[nf], nib_mask);
            }
            // keep the scale a plain fp32 register: otherwise the compiler folds
            // the fp16 conversion into v_fma_mix_f32 for every scale FMA, which
            // issues slower and raises register pressure into spills
            asm volatile("" : "+v"(dv[nf]));
        }
        // every slot fragment, unconditionally (rows past the count are computed
        // and dropped at the store): per-fragment branches cost registers and
        // serialise the schedule
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
            const u32x4 a =
                *(const u32x4*)(Sa + blk * AROWS * 64 + (mf * 16 + l16) * 64 + swz);
            const f32x4 c = *(const f32x4*)&Sc[blk * AROWS + mf * 16 + 4 * g];
            f32x4 t[NF];
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) t[nf] = mfma_bf16(a, bq[nf], c);
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mf][nf][i] = fmaf(dv[nf], t[nf][i], acc[mf][nf][i]);
        }
    }
}

// Tile lookup.  Slot tiles cover an expert's slots MT at a time (the last one
// partial); each has n_tiles column tiles.
// The grid is an upper bound, so the numbering is made once the real counts
// are known; the column tiles of one slot tile always take consecutive block
// numbers of one XCD (blocks congruent to x mod 8 run on XCD x), so they share
// that XCD's L2.
//
//  * Many workgroups (more than FFN_MFMA_LPT_UNITS): slot tiles in expert
//    order, the sequence of workgroups cut into 8 equal runs, run x for XCD
//    x, so the next slot tile of the same expert also shares the XCD's L2 (its
//    weights).  An expert's tiles hold MT slots each but the last, which takes
//    up to mtx: a remainder of at most mtx - MT slots joins the tile before it
//    instead of streaming the expert's weights once more for a few slots.
//  * Few (a grid of about three rounds of resident workgroups or less, as with
//    a few hundred tokens over many experts): how long the kernel takes is
//    decided by how the tiles pack, and a tile's time grows with its slot
//    count.  Slot tiles are ranked longest first (97-128 slots, then 65-96,
//    33-64, 1-32; expert order within a class) and rank r goes to XCD r mod 8,
//    so every XCD starts its long tiles first and the short ones fill in.
//    A light slot tile (at most 32 slots) here has 2 n_tiles half-width
//    column tiles: it streams the same weight bytes as a full tile for a
//    quarter of the products, so it runs almost as long, and halving its
//    columns halves the granule that the last round packs.
//
// Wave 0 scans the expert counts (up to 4 experts per lane); returns false
// for a workgroup without a tile.  half: ntile counts half-width column tiles.
constexpr int FFN_MFMA_LPT_UNITS = 1536;
constexpr int FFN_MFMA_LIGHT = 32;  // slot tiles of at most this many slots are light

MOE_DEV int tile_class(int size) { return size > 96 ? 0 : size > 64 ? 1 : size > FFN_MFMA_LIGHT ? 2 : 3; }

MOE_DEV int scan_incl(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}

__device__ bool find_tile(const int32_t* __restrict__ offsets, int E, int bid, int n_tiles, int mtx,
                          int* s_res, int& e_out, int& base, int& cnt, int& ntile, bool& half) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int c[4], full[4], rem[4], u[4], tot = 0;
        int nm[4], um[4], totm = 0;  // slot tiles with a merged last tile, their units
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane * 4 + q;
            c[q] = e < E ? offsets[e + 1] - offsets[e] : 0;
            full[q] = c[q] / MT;
            rem[q] = c[q] - full[q] * MT;
            u[q] = (full[q] + (rem[q] ? 1 : 0)) * n_tiles;  // column tiles
            tot += u[q];
            nm[q] = c[q] <= mtx ? (c[q] > 0 ? 1 : 0) : 1 + (c[q] - mtx + MT - 1) / MT;
            um[q] = nm[q] * n_tiles;
            totm += um[q];
        }
        const int incl = scan_incl(tot, lane);
        const int total = __shfl(incl, 63);  // workgroups with a tile
        // this lane's find: expert, its slot tile, column tile
        int e_sel = -1, k_sel = 0, c_sel = 0, nt_sel = 0, n_sel = 0;
        const bool many = total > FFN_MFMA_LPT_UNITS;
        if (many) {
            // tiles of MT slots, the last of up to mtx
            const int inclm = scan_incl(totm, lane);
            const int totalm = __shfl(inclm, 63);
            const int per_xcd = (totalm + 7) >> 3;
            const int lin = (bid & 7) * per_xcd + (bid >> 3);
            const bool have = (bid >> 3) < per_xcd && lin < totalm;
            int run = inclm - totm;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (have && lin >= run && lin < run + um[q]) {
                    const int ue = lin - run;
                    e_sel = lane * 4 + q;
                    c_sel = c[q];
                    n_sel = nm[q];
                    k_sel = ue / n_tiles;
                    nt_sel = ue - k_sel * n_tiles;
                }
                run += um[q];
            }
        } else {
            // tiles per class: class 0 holds an expert's full tiles and a
            // remainder of 97-127 slots, classes 1-3 the remainder (if any)
            int n0[4], rc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cls = rem[q] ? tile_class(rem[q]) : -1;
                n0[q] = full[q] + (cls == 0 ? 1 : 0);
                rc[q] = cls > 0 ? cls : -1;
            }
            auto lane_count = [&](int k) {
                int s = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) s += k == 0 ? n0[q] : (rc[q] == k ? 1 : 0);
                return s;
            };
            // inclusive scans of the class counts, two 16-bit fields per int (in
            // this branch a class holds at most FFN_MFMA_LPT_UNITS tiles)
            const int s01 = scan_incl(lane_count(0) + (lane_count(1) << 16), lane);
            const int s23 = scan_incl(lane_count(2) + (lane_count(3) << 16), lane);
            const int a01 = __shfl(s01, 63), a23 = __shfl(s23, 63);
            const int tot0 = a01 & 0xFFFF, tot1 = a01 >> 16, tot2 = a23 & 0xFFFF, tot3 = a23 >> 16;
            const int R = tot0 + tot1 + tot2 + tot3, T012 = tot0 + tot1 + tot2;
            // XCD x takes ranks x, x + 8, ...: its first c012 of them are of
            // classes 0-2 (n_tiles units each), the rest light (2 n_tiles)
            const int x = bid & 7, qpos = bid >> 3;
            const int c012 = T012 > x ? (T012 - x + 7) >> 3 : 0;
            int i, nt;
            if (qpos < c012 * n_tiles) {
                i = qpos / n_tiles;
                nt = qpos - i * n_tiles;
            } else {
                const int q2 = qpos - c012 * n_tiles;
                const int j = q2 / (2 * n_tiles);
                i = c012 + j;
                nt = q2 - j * 2 * n_tiles;
            }
            const int r = x + 8 * i;  // rank of this block's slot tile
            if (r < R) {
                const int k = r < tot0 ? 0 : r < tot0 + tot1 ? 1 : r < T012 ? 2 : 3;
                const int idx = r - (k >= 1 ? tot0 : 0) - (k >= 2 ? tot1 : 0) - (k >= 3 ? tot2 : 0);
                const int inclk = k == 0 ? (s01 & 0xFFFF) : k == 1 ? (s01 >> 16)
                                : k == 2 ? (s23 & 0xFFFF) : (s23 >> 16);
                int run = inclk - lane_count(k);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nq = k == 0 ? n0[q] : (rc[q] == k ? 1 : 0);
                    if (idx >= run && idx < run + nq) {
                        e_sel = lane * 4 + q;
                        // class 0: the (idx - run)-th tile of the expert; others: its remainder
                        k_sel = k == 0 ? idx - run : full[q];
                        c_sel = c[q];
                        nt_sel = nt;
                    }
                    run += nq;
                }
            }
        }
        if (e_sel >= 0) {
            s_res[0] = e_sel;
            s_res[1] = offsets[e_sel] + k_sel * MT;
            s_res[2] = many ? (k_sel == n_sel - 1 ? c_sel - k_sel * MT : MT) : min(MT, c_sel - k_sel * MT);
            s_res[3] = nt_sel;
            s_res[4] = !many && c_sel - k_sel * MT <= FFN_MFMA_LIGHT;
        }
        // exactly one lane finds the tile; without one lane 63 marks the block
        // (the whole wave votes)
        const bool found = __ballot(e_sel >= 0) != 0;
        if (lane == 63 && !found) s_res[0] = -1;
    }
    __syncthreads();
    e_out = s_res[0];
    base = s_res[1];
    cnt = s_res[2];
    ntile = s_res[3];
    half = s_res[4] != 0;
    return e_out >= 0;
}

// MODE 0: gate/up.  act = staged x [T][apitch] (rows gathered through the
//         slots' tokens), csum = -1.5 * block sums per token [T][H/32]
//         (cs_row = H/32, cs_blk = 1), W = w_gate_up, rows_e = 2I, ncols = I;
//         writes h (slot order, rows hpitch apart) and its block sums
//         block-major [I/32][hs_blk = N].
// MODE 1: down.     act = h [N][apitch], csum = its block sums [I/32][N]
//         (cs_row = 1, cs_blk = N), W = w_down, rows_e = ncols = H; writes
//         y_sorted.
// Sum (row, block) is at csum[row * cs_row + block * cs_blk].
// Requires an even number of blocks per row (H and I multiples of 64), so that
// every pair of blocks starts on a dword boundary.
//
// Tile: MT slots x NT weight rows; wave w owns weight rows 64w..64w+63 of the
// tile (4 MFMA row fragments) against all MT slots (8 fragments), 128 fp32
// accumulators per lane.
//
// Every operand goes through LDS by direct loads (buffer loads with the lds
// modifier), two stages in turn: iteration j issues the loads of pair j+1 into
// the stage pair j-1 used, runs the MFMAs of pair j, waits for its own loads
// and ends on a barrier, so no register holds staged data.  A stage is the
// activations [2 blocks][MT rows][64 B] (the 16-byte chunks of a row rotated
// by (row >> 2) & 3, so the fragment reads are conflict-free), their block sums
// [2][MT] and the tile's weight rows [NT][48 B] (a row's 36 bytes of the pair
// as its bytes 0-15, 16-31 and 20-35: direct loads of 12 bytes would land 16
// bytes apart, so three 16-byte loads that never cross the pair).  The loads
// are issued by dma16/dma4, so the only waits for them are the kernel's own:
// each step waits until the next pair's loads have landed (later pairs stay in
// flight) and ends on a bare s_barrier after an LDS-only wait (a memory-model
// fence would also drain the direct loads).
// Per wave and pair: MF/2 16-byte loads of activations (16 rows of one block
// each), one 4-byte load of block sums (64 rows of one block) and three
// 16-byte loads of weights (21 rows per instruction), in place of eight
// per-lane weight loads that each touched 16 rows.  A third weight stage (two
// pairs in flight) measured no faster for full tiles; tiles of at most 32
// slots, which have a quarter of the work per pair, run a three-stage ring
// (a fourth stage measured no faster).
//
// BUF: the activation buffer spans less than 2 GiB (its block sums and one
// expert's weights are smaller still), so every offset fits a signed 32-bit
// lane offset.  The direct loads are then buffer loads: a resource per buffer
// in scalar registers, a fixed offset per lane and the pair's offset as a
// scalar operand, so a load costs no vector address arithmetic (otherwise
// every load and pair adds a 64-bit address).
template <int MODE, bool BUF>
__global__ __launch_bounds__(256) void ffn_mfma(
    const uint16_t* __restrict__ act, const float* __restrict__ csum, const uint8_t* __restrict__ W,
    int nb, int apitch, int rows_e, int ncols, int cs_row, int cs_blk, int hpitch, int hs_blk,
    int n_tiles,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, int K, int E, uint16_t* __restrict__ h_out,
    float* __restrict__ hsum_out, float* __restrict__ y_out) {
    __shared__ __attribute__((aligned(16))) uint8_t a0[2 * MTX * 64], a1[2 * MTX * 64];
    __shared__ __attribute__((aligned(16))) float cc0[2 * MTX], cc1[2 * MTX];
    __shared__ __attribute__((aligned(16))) uint8_t w0[NT * 48], w1[NT * 48];
    // the third stage of the light ring (tiles of at most 32 slots) lives in the
    // parts of stage 0's activation and sum arrays that a light tile leaves free
    static_assert(2 * 32 * 64 + 2 * 32 * 64 + NT * 48 <= 2 * MTX * 64 && 2 * 32 + 2 * 32 <= 2 * MTX,
                  "light third stage fits");
    struct StageRef {
        uint8_t* a;
        float* c;
        uint8_t* w;
    };
    StageRef st0{a0, cc0, w0}, st1{a1, cc1, w1};
    __shared__ int s_res[5];

    int e, base, cnt, ntile;
    bool half;
    // the merged last tile (up to MTX slots) only where the loads are buffer
    // loads: the 64-bit-address variant would exceed 256 VGPRs with its 10
    // fragments (and run one wave per SIMD)
    constexpr int MX = BUF ? MTX : MT;
    if (!find_tile(offsets, E, blockIdx.x, n_tiles, MX, s_res, e, base, cnt, ntile, half)) return;
    e = __builtin_amdgcn_readfirstlane(e);
    base = __builtin_amdgcn_readfirstlane(base);
    cnt = __builtin_amdgcn_readfirstlane(cnt);
    ntile = __builtin_amdgcn_readfirstlane(ntile);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const uint32_t rowbytes = (uint32_t)nb * 18u;
    const uint8_t* We = W + (size_t)e * rows_e * rowbytes;
    const int npairs = nb >> 1;

    // byte offset in csum of entry P of a stage's block sums [2 blocks][rows]
    auto sum_byte = [&](int P, int rows) -> int64_t {
        const int blk = P / rows, r = P - blk * rows;
        const int p = base + min(r, cnt - 1);
        const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
        return (arow * cs_row + (int64_t)blk * cs_blk) * 4;
    };
    // buffer resources (unbounded: every offset stays inside its buffer)
    const i32x4 r_act = buffer_rsrc(act), r_cs = buffer_rsrc(csum), r_w = buffer_rsrc(We);

    const int mfa = min(MX / 16, (cnt + 15) >> 4);  // valid slot fragments

    // The main loop and epilogue for MF slot fragments (16 slots each).  A tile
    // of at most 32, 64 or 96 slots (an expert's last, partial tile, or a small
    // expert) runs with MF = 2, 4 or 6: a quarter, half or three quarters of
    // the activation loads, MFMAs and scale FMAs of a full tile.
    auto run = [&](auto mf_const, auto nf_const) {
        constexpr int MF = decltype(mf_const)::value;
        // activation loads per wave per pair: the workgroup's 2 MF, the last one
        // repeated by a wave past them (MF = 9)
        constexpr int NA = (2 * MF + 3) / 4;
        constexpr bool LIGHT = MF == 2;
        constexpr bool WIDE = MF > MT / 16;  // a merged last tile of more than MT slots
        constexpr int AROWS = LIGHT ? 32 : WIDE ? MTX : MT;  // rows per block in a stage
        // 16-row weight fragments per wave: 4, or 2 in a light tile's
        // half-width column tiles
        constexpr int NF = decltype(nf_const)::value;
        constexpr int NWL = (48 * NF + 63) / 64;  // 16-byte weight loads per wave per pair

        // ---- this wave's weight rows ----
        // MODE 0: hidden columns c0 .. c0 + 8 NF - 1 (gate rows, then the same
        //         rows of up)
        // MODE 1: output rows c0 .. c0 + 16 NF - 1
        const int c0 = MODE == 0 ? ntile * (32 * NF) + 8 * NF * wave : ntile * (64 * NF) + 16 * NF * wave;
        int nfa;  // valid row fragments (whole wave for MODE 0)
        if (MODE == 0)
            nfa = c0 < ncols ? NF : 0;
        else
            nfa = max(0, min(NF, (ncols - c0) >> 4));
        const bool active = nfa > 0;
        // weight pieces: a row's 36 bytes of a pair as three 16-byte loads of its
        // bytes 0-15, 16-31 and 20-35 (never past the pair), 48 bytes per row in
        // LDS; lane piece i of a pair is q = 64 i + lane of the wave's 48 NF
        // pieces (lanes past them repeat the last one), row 16 nf + l16 = q / 3
        // of the wave, piece q % 3
        uint32_t woff[NWL];
#pragma unroll
        for (int i = 0; i < NWL; ++i) {
            const int q = min(64 * i + lane, 48 * NF - 1), r = q / 3;
            const int nf = r >> 4, rl = r & 15;
            int row;
            if (MODE == 0)
                row = min(c0 + (nf % (NF / 2)) * 16 + rl, ncols - 1) + (nf / (NF / 2)) * ncols;
            else
                row = min(c0 + nf * 16 + rl, rows_e - 1);
            const int pc = q % 3;
            woff[i] = (uint32_t)row * rowbytes + (pc == 0 ? 0u : pc == 1 ? 16u : 20u);
        }

        f32x4 acc[MF][NF];
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int jn = 0; jn < NF; ++jn) acc[i][jn] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // activation loads: the WG's 2 MF instructions t = NA w + i cover block
        // t / MF, rows 16 (t % MF) .. +15; lane: row + (lane >> 2), LDS chunk
        // position lane & 3 holding the row's chunk (lane & 3) ^ ((row >> 2) & 3)
        int64_t abyte[NA];  // byte offsets in act
        int adst[NA];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int t = min(NA * wave + i, 2 * MF - 1), blk = t / MF, rg = t % MF;
            const int r = 16 * rg + (lane >> 2);
            const int p = base + min(r, cnt - 1);
            const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
            const int chunk = (lane & 3) ^ ((r >> 2) & 3);
            abyte[i] = (arow * apitch + blk * 32 + 8 * chunk) * 2;
            adst[i] = blk * AROWS * 64 + rg * 1024;
        }
        // block sums: a heavy stage takes entries 64 w + lane from wave w (block
        // w >> 1 of rows 64 (w & 1) + lane when AROWS = MT), and in a wide one
        // wave 0 also entries 2 AROWS - 64 + lane (the last rows of block 1,
        // where the two overlap the same sums); a light stage its 2 x 32 sums
        // (block lane >> 5, row lane & 31) from every wave alike (the same
        // bytes, so the four copies agree)
        int64_t cbyte = sum_byte(64 * wave + lane, AROWS);
        const int64_t cbyte_x = WIDE ? sum_byte(2 * AROWS - 64 + lane, AROWS) : 0;
        int cdst = 64 * wave;
        if constexpr (LIGHT) {
            const int r = lane & 31;
            const int p = base + min(r, cnt - 1);
            const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
            cbyte = (arow * cs_row + (int64_t)(lane >> 5) * cs_blk) * 4;
            cdst = 0;
        }
        // pair j: activations 128 bytes, block sums two blocks (2 cs_blk
        // floats) and weights 36 bytes further on
        const int cpair = 8 * cs_blk;
        // A wave without weight rows (the last gate/up column tile when I is not
        // a multiple of 128) still loads its share of the activations, which
        // the other waves read, but not its weights, which nobody reads; the
        // light ring keeps them, since its waits count every wave's loads alike.
        const bool wload = LIGHT || active;
        auto issue = [&](const StageRef& S, int j) {
            if constexpr (BUF) {
#pragma unroll
                for (int i = 0; i < NA; ++i) dma16(S.a + adst[i], (uint32_t)abyte[i], r_act, 128u * j);
                dma4(S.c + cdst, (uint32_t)cbyte, r_cs, (uint32_t)(cpair * j));
                if (WIDE && wave == 0)
                    dma4(S.c + 2 * AROWS - 64, (uint32_t)cbyte_x, r_cs, (uint32_t)(cpair * j));
                if (wload) {
#pragma unroll
                    for (int i = 0; i < NWL; ++i) dma16(S.w + 64 * 48 * wave + 1024 * i, woff[i], r_w, 36u * j);
                }
            } else {
                const uint8_t* act_b = reinterpret_cast<const uint8_t*>(act);
                const uint8_t* cs_b = reinterpret_cast<const uint8_t*>(csum);
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    __builtin_amdgcn_global_load_lds((glb_void_t*)(act_b + abyte[i] + 128 * j),
                                                     (lds_void_t*)(S.a + adst[i]), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((glb_void_t*)(cs_b + cbyte + (int64_t)cpair * j),
                                                 (lds_void_t*)(S.c + cdst), 4, 0, 0);
                if (WIDE && wave == 0)
                    __builtin_amdgcn_global_load_lds((glb_void_t*)(cs_b + cbyte_x + (int64_t)cpair * j),
                                                     (lds_void_t*)(S.c + 2 * AROWS - 64), 4, 0, 0);
                if (wload) {
#pragma unroll
                    for (int i = 0; i < NWL; ++i)
                        __builtin_amdgcn_global_load_lds(
                            (glb_void_t*)(We + woff[i] + 36u * (uint32_t)j),
                            (lds_void_t*)(S.w + 64 * 48 * wave + 1024 * i), 16, 0, 0);
                }
            }
        };
        const int swz = 16 * (g ^ ((l16 >> 2) & 3));  // this lane's chunk position in a row
        const int q1off = g < 3 ? 20 + 4 * g : 44;     // qs1 dword g in a row's 48 bytes
        // the nibble mask in a VGPR: each unpacking step is then a shift and a
        // v_and_or_b32 (a VOP3 operation takes no literal on gfx950)
        uint32_t nib_mask;
        asm volatile("v_mov_b32 %0, 0x00780078" : "=v"(nib_mask));
        auto compute = [&](const StageRef& S) {
            stage_products<MF, NF, AROWS>(S.a, S.c, S.w + (wave * 64 + l16) * 48, g, l16, swz, q1off, nib_mask,
                                          acc);
        };
        // One step per pair: issue the loads of a later pair (none past the
        // last), compute this pair, wait for this wave's loads of the next pair,
        // barrier.
        if constexpr (LIGHT) {
            // three stages (the third in arrays of its own): step j issues pair
            // j+2 into the stage pair j-1 used and waits for pair j+1 (issued a
            // step earlier)
            const StageRef st2{a0 + 2 * 32 * 64, cc0 + 2 * 32, a0 + 2 * 2 * 32 * 64};
            constexpr int OPS = NA + 1 + NWL;  // direct loads per wave per pair
            auto step = [&](const StageRef& cur, const StageRef& nxt, int j) {
                const bool more = j + 2 < npairs;
                if (more) issue(nxt, j + 2);
                if (active) compute(cur);
                if (more)
                    wait_vmcnt<OPS>();
                else
                    wait_vmcnt<0>();
                stage_barrier();
            };
            issue(st0, 0);
            if (npairs > 1) {
                issue(st1, 1);
                wait_vmcnt<OPS>();
            } else {
                wait_vmcnt<0>();
            }
            stage_barrier();
            for (int j = 0; j < npairs; j += 3) {
                step(st0, st2, j);
                if (j + 1 < npairs) step(st1, st0, j + 1);
                if (j + 2 < npairs) step(st2, st1, j + 2);
            }
        } else {
            // two stages: step j issues pair j+1 into the stage pair j-1 used
            // and waits for it before the barrier
            auto step = [&](const StageRef& cur, const StageRef& nxt, int j) {
                if (j + 1 < npairs) issue(nxt, j + 1);
                if (active) compute(cur);
                wait_vmcnt<0>();
                stage_barrier();
            };
            issue(st0, 0);
            wait_vmcnt<0>();
            stage_barrier();
            for (int j = 0; j < npairs; j += 2) {
                step(st0, st1, j);
                if (j + 1 < npairs) step(st1, st0, j + 1);
            }
        }
        // The last step issues nothing, waits for all of its wave's loads and
        // ends on the barrier: the stage arrays are free for the epilogues.
        if (!active) return;
        if constexpr (MODE == 0 && NF == 2) {
            // A light tile's half-width column tile: waves 2k and 2k+1 hold
            // columns 0-15 and 16-31 of h block c0 >> 5.  Each writes its h values
            // into the pair's staging rows and its 16-column row sums to LDS; after
            // a barrier the even wave adds the two halves (columns 0-15 first) and
            // stores the rows.  The four waves are active together or not at all
            // (I is a multiple of 64, the width of the tile), so all reach the
            // barrier.
            const int hblk = c0 >> 5, half = wave & 1;
            constexpr int RB = 80;
            static_assert(32 * RB <= 2 * MT * 64 && 4 * 32 * 4 <= NT * 48, "light h staging fits");
            uint8_t* R = (wave >> 1) ? a1 : a0;
            float* psum = reinterpret_cast<float*>(w0);  // [wave][row]
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                if (mf < mfa) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = mf * 16 + 4 * g + i;
                        const float gv = 16.f * acc[mf][0][i], uv = 16.f * acc[mf][1][i];
                        const uint16_t hb = f32_to_bf16(gelu_tanh(gv) * uv);
                        float s = bf16_to_f32(hb);
                        *(uint16_t*)(R + r * RB + 2 * perm_pos(half * 16 + l16)) = hb;
                        s += dpp_mov_f32<DPP_QUAD_XOR1>(s);
                        s += dpp_mov_f32<DPP_QUAD_XOR2>(s);
                        s += dpp_mov_f32<DPP_ROW_HALF_MIRROR>(s);
                        s += dpp_mov_f32<DPP_ROW_MIRROR>(s);
                        if (l16 == 0) psum[wave * 32 + r] = s;
                    }
                }
            }
            __syncthreads();
            if (half == 0) {
#pragma unroll
                for (int mf = 0; mf < MF; ++mf) {
                    if (mf < mfa) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = mf * 16 + 4 * g + i;
                            if (r < cnt && l16 == 0)
                                hsum_out[(int64_t)hblk * hs_blk + base + r] =
                                    -1.5f * (psum[wave * 32 + r] + psum[(wave + 1) * 32 + r]);
                        }
                        const int r = mf * 16 + (lane >> 2), ch = lane & 3;
                        const uint4 v = *(const uint4*)(R + r * RB + 16 * ch);
                        if (r < cnt) *(uint4*)(h_out + (int64_t)(base + r) * hpitch + hblk * 32 + 8 * ch) = v;
                    }
                }
            }
        } else if constexpr (MODE == 0) {
            // h = GELU(g) * u for hidden columns c0 .. c0+31: one Q4_0 block of the
            // down product's K, written in the MFMA order with its sum.  Each slot
            // fragment's 16 rows of 64 bytes go through a stage array of the wave's
            // own (rows 80 bytes apart, so the 4 lane groups' writes fall in
            // different banks; fragments 8 and 9 reuse the rows of fragments 0 and
            // 1) and leave as one 16-byte store per lane.
            const int hblk = c0 >> 5;
            constexpr int RB = 80;
            static_assert(MT * RB <= NT * 48 && NT * 48 <= 2 * MTX * 64, "h staging fits");
            uint8_t* R = wave == 0 ? a0 : wave == 1 ? a1 : wave == 2 ? w0 : w1;
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                if (mf < mfa) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = mf * 16 + 4 * g + i;
                        const bool ok = r < cnt;
                        const int64_t p = base + min(r, cnt - 1);
                        float s = 0.f;
#pragma unroll
                        for (int f = 0; f < 2; ++f) {
                            const float gv = 16.f * acc[mf][f][i], uv = 16.f * acc[mf][2 + f][i];
                            const uint16_t hb = f32_to_bf16(gelu_tanh(gv) * uv);
                            s += bf16_to_f32(hb);
                            *(uint16_t*)(R + (r & (MT - 1)) * RB + 2 * perm_pos(f * 16 + l16)) = hb;
                        }
                        // sum over the 16 lanes holding this row's columns
                        s += dpp_mov_f32<DPP_QUAD_XOR1>(s);
                        s += dpp_mov_f32<DPP_QUAD_XOR2>(s);
                        s += dpp_mov_f32<DPP_ROW_HALF_MIRROR>(s);
                        s += dpp_mov_f32<DPP_ROW_MIRROR>(s);
                        if (ok && l16 == 0) hsum_out[(int64_t)hblk * hs_blk + p] = -1.5f * s;
                    }
                    const int r = mf * 16 + (lane >> 2), ch = lane & 3;
                    const uint4 v = *(const uint4*)(R + (r & (MT - 1)) * RB + 16 * ch);
                    if (r < cnt) *(uint4*)(h_out + (int64_t)(base + r) * hpitch + hblk * 32 + 8 * ch) = v;
                }
            }
        } else {
            // y through LDS: two slot fragments at a time, a wave turns its 32 slots
            // x 64 columns (fp32) from the MFMA layout (a lane holds 4 slots of one
            // column) into rows in a stage array of its own (rows 68 floats apart, so
            // the 4 lane groups' writes fall in different banks), then writes each
            // slot's 256 bytes as 16-byte stores (one instruction covers 4 rows
            // instead of 4 rows x 16 columns of 4-byte stores)
            const int H = ncols;
            constexpr int RS = 68;
            static_assert(32 * RS * 4 <= NT * 48 && NT * 48 <= 2 * MTX * 64, "y staging fits");
            float* R = reinterpret_cast<float*>(wave == 0 ? a0 : wave == 1 ? a1 : wave == 2 ? w0 : w1);
            const int cq = lane & 15;
#pragma unroll
            for (int m2 = 0; m2 < MF; m2 += 2) {
                if (m2 < mfa) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        if (m2 + h < MF)  // MF = 9: the last pair is one fragment
#pragma unroll
                            for (int nf = 0; nf < NF; ++nf)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    R[(16 * h + 4 * g + i) * RS + 16 * nf + l16] = 16.f * acc[m2 + h][nf][i];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int rl = 4 * q + (lane >> 4), r = 16 * m2 + rl;
                        const float4 v = *reinterpret_cast<const float4*>(R + rl * RS + 4 * cq);
                        if (r < cnt && cq < 4 * nfa)
                            *reinterpret_cast<float4*>(y_out + (int64_t)(base + r) * H + c0 + 4 * cq) = v;
                    }
                }
            }
        }
    };
    using F2 = std::integral_constant<int, 2>;
    using F4 = std::integral_constant<int, 4>;
    if (cnt <= 32) {
        if (half)
            run(std::integral_constant<int, 2>{}, F2{});
        else
            run(std::integral_constant<int, 2>{}, F4{});
    } else if (cnt <= 64) {
        run(std::integral_constant<int, 4>{}, F4{});
    } else if (cnt <= 96) {
        run(std::integral_constant<int, 6>{}, F4{});
    } else if (!BUF || cnt <= MT) {
        run(std::integral_constant<int, 8>{}, F4{});
    } else if constexpr (BUF) {
        if (cnt <= 144)
            run(std::integral_constant<int, 9>{}, F4{});
        else
            run(std::integral_constant<int, MTX / 16>{}, F4{});
    }
}

// Activations -> MFMA block order (rows pitch apart), plus -1.5 * block sums
// ([T][nb]).  Four lanes per 32-element block, one 16-byte quarter each (loads
// and stores of a wave are contiguous): output chunk c of a block holds
// elements 4c..4c+3 of quarter c >> 1 and elements 4c+16..4c+19 of quarter
// (c >> 1) + 2, which reach lane c through quad DPP moves.  The block sum is
// each lane's 8 values in order, then the quad's four partial sums.
__global__ __launch_bounds__(256) void ffn_mfma_prep(const uint16_t* __restrict__ x, int64_t T, int nb,
                                                     int pitch, uint16_t* __restrict__ xp,
                                                     float* __restrict__ xs) {
    const int64_t nblocks = T * nb;
    const int64_t nq = nblocks * 4;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[min(q, nq - 1)];
    const int c = threadIdx.x & 3;
    float s = 0.f;
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s += __uint_as_float(w4[i] << 16);
        s += __uint_as_float(w4[i] & 0xFFFF0000u);
    }
    s += dpp_mov_f32<DPP_QUAD_XOR1>(s);
    s += dpp_mov_f32<DPP_QUAD_XOR2>(s);
    constexpr int FROM_LO = 0x50;  // quad_perm [0,0,1,1]: lane c reads lane c >> 1
    constexpr int FROM_HI = 0xFA;  // quad_perm [2,2,3,3]: lane c reads lane (c >> 1) + 2
    auto mv = [](uint32_t a, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp((int)a, (int)a, decltype(ctrl)::value, 0xF, 0xF, false);
    };
    using LO = std::integral_constant<int, FROM_LO>;
    using HI = std::integral_constant<int, FROM_HI>;
    const bool odd = c & 1;
    // A = elements (4c, 4c+1), B = (4c+2, 4c+3), C = (4c+16, 4c+17), D = (4c+18, 4c+19)
    const uint32_t a0 = mv(v.x, LO{}), b0 = mv(v.y, LO{}), a1 = mv(v.z, LO{}), b1 = mv(v.w, LO{});
    const uint32_t c0 = mv(v.x, HI{}), d0 = mv(v.y, HI{}), c1 = mv(v.z, HI{}), d1 = mv(v.w, HI{});
    const uint32_t A = odd ? a1 : a0, B = odd ? b1 : b0, C = odd ? c1 : c0, D = odd ? d1 : d0;
    u32x4 o;
    o.x = (A & 0xFFFFu) | (B << 16);
    o.y = (C & 0xFFFFu) | (D << 16);
    o.z = (A >> 16) | (B & 0xFFFF0000u);
    o.w = (C >> 16) | (D & 0xFFFF0000u);
    if (q < nq) {
        const int64_t t = q / (4 * nb), qq = q - t * 4 * nb;
        reinterpret_cast<u32x4*>(xp + t * pitch)[qq] = o;
        if (c == 0) xs[q >> 2] = -1.5f * s;
    }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Grid of a grouped-GEMM launch over at most mtiles slot tiles: room for
// ceil(mtiles / 8) slot tiles per XCD with all their column tiles, and, when
// the longest-first numbering is possible (at most FFN_MFMA_LPT_UNITS column
// tiles in all), for its half-width light column tiles.
static int mfma_grid(int mtiles, int n_tiles) {
    const int g_many = (mtiles + 7) / 8 * 8 * n_tiles;
    const int r_few = std::min(mtiles, FFN_MFMA_LPT_UNITS / n_tiles);
    const int g_few = (r_few + 7) / 8 * 8 * 2 * n_tiles;
    return std::max(g_many, g_few);
}

}  // namespace

// Row pitch (elements) of a staged activation matrix with `cols` bf16 columns
// (a multiple of 64): an odd number of 128-byte lines.  Tiles gather rows of
// one block pair at a time; with an even line count (5,632 bytes for 2,816
// columns: 44 lines) those rows fall on a quarter of the L2 channels.
static int act_pitch(int cols) { return ((cols * 2 / 128) & 1) ? cols : cols + 64; }

size_t ffn_mfma_ws_bytes(int64_t T, int H, int I, int64_t N) {
    return align256((size_t)T * act_pitch(H) * 2) + align256((size_t)T * (H / 32) * 4) +
           align256((size_t)N * act_pitch(I) * 2) + align256((size_t)N * (I / 32) * 4);
}

// Buffer loads take 32-bit offsets: every byte of an activation buffer of this
// size (its block sums are a sixteenth of it, one expert's weights at most
// 2 x MOE_MAX_I rows of MOE_MAX_H / 32 blocks) is reachable.
static bool buf_ok(size_t act_bytes) { return act_bytes < ((size_t)1 << 31); }

hipError_t launch_ffn_mfma(const void* x, int64_t T, int H, const uint8_t* w_gate_up,
                           const uint8_t* w_down, int I, int E, int K, int N,
                           const int32_t* offsets, const int32_t* sorted_slots, void* ws,
                           float* y_sorted, hipStream_t st) {
    uint8_t* p = (uint8_t*)ws;
    const int xpitch = act_pitch(H), hpitch = act_pitch(I);
    uint16_t* xp = (uint16_t*)p;
    p += align256((size_t)T * xpitch * 2);
    float* xs = (float*)p;
    p += align256((size_t)T * (H / 32) * 4);
    uint16_t* hp = (uint16_t*)p;
    p += align256((size_t)N * hpitch * 2);
    float* hs = (float*)p;

    const int64_t nblk = T * (H / 32);
    ffn_mfma_prep<<<(unsigned)((4 * nblk + 255) / 256), 256, 0, st>>>((const uint16_t*)x, T, H / 32, xpitch,
                                                                      xp, xs);

    // slot tiles: sum over experts of ceil(count / MT) <= N / MT + (experts hit);
    // the workgroups past the real count exit at once
    const int mtiles = N / MT + min(E, N);
    {
        const int n_tiles = (I + NT / 2 - 1) / (NT / 2);
        const int total = mfma_grid(mtiles, n_tiles);
        if (buf_ok((size_t)T * xpitch * 2))
            ffn_mfma<0, true><<<total, 256, 0, st>>>(xp, xs, w_gate_up, H / 32, xpitch, 2 * I, I, H / 32, 1,
                                                     hpitch, N, n_tiles, offsets, sorted_slots, K, E, hp,
                                                     hs, nullptr);
        else
            ffn_mfma<0, false><<<total, 256, 0, st>>>(xp, xs, w_gate_up, H / 32, xpitch, 2 * I, I, H / 32, 1,
                                                      hpitch, N, n_tiles, offsets, sorted_slots, K, E, hp,
                                                      hs, nullptr);
    }
    {
        const int n_tiles = (H + NT - 1) / NT;
        const int total = mfma_grid(mtiles, n_tiles);
        if (buf_ok((size_t)N * hpitch * 2))
            ffn_mfma<1, true><<<total, 256, 0, st>>>(hp, hs, w_down, I / 32, hpitch, H, H, 1, N, 0, 0,
                                                     n_tiles, offsets, sorted_slots, K, E, nullptr, nullptr,
                                                     y_sorted);
        else
            ffn_mfma<1, false><<<total, 256, 0, st>>>(hp, hs, w_down, I / 32, hpitch, H, H, 1, N, 0, 0,
                                                      n_tiles, offsets, sorted_slots, K, E, nullptr,
                                                      nullptr, y_sorted);
    }
    return hipGetLastError();
}

size_t linear_mfma_ws_bytes(int64_t T, int H) {
    return align256((size_t)T * act_pitch(H) * 2) + align256((size_t)T * (H / 32) * 4);
}

hipError_t launch_linear_mfma(const void* x, int64_t T, int H, const uint8_t* W, int R,
                              const int32_t* offsets, const int32_t* slots, void* ws, float* y,
                              hipStream_t st) {
    const int xpitch = act_pitch(H);
    uint16_t* xp = (uint16_t*)ws;
    float* xs = (float*)((uint8_t*)ws + align256((size_t)T * xpitch * 2));
    const int64_t nblk = T * (H / 32);
    ffn_mfma_prep<<<(unsigned)((4 * nblk + 255) / 256), 256, 0, st>>>((const uint16_t*)x, T, H / 32, xpitch,
                                                                      xp, xs);
    const int N = (int)T, mtiles = N / MT + 1;
    const int n_tiles = (R + NT - 1) / NT;
    const int total = mfma_grid(mtiles, n_tiles);
    if (buf_ok((size_t)T * xpitch * 2))
        ffn_mfma<1, true><<<total, 256, 0, st>>>(xp, xs, W, H / 32, xpitch, R, R, H / 32, 1, 0, 0,
                                                 n_tiles, offsets, slots, 1, 1, nullptr, nullptr, y);
    else
        ffn_mfma<1, false><<<total, 256, 0, st>>>(xp, xs, W, H / 32, xpitch, R, R, H / 32, 1, 0, 0,
                                                  n_tiles, offsets, slots, 1, 1, nullptr, nullptr, y);
    return hipGetLastError();
}

}  // namespace moe
