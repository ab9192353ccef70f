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
// slots x 64 rows (8 x 4 MFMA tiles); two Q4_0 blocks per stage.  For gate/up
// a wave's 64 rows are 32 gate rows and the 32 up rows of the same hidden
// columns, so each lane holds gate and up of the same (slot, column) in
// matching registers and GELU(g) * u is formed in the epilogue.
#include <type_traits>

#include "kernels.h"

namespace moe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MT = 128;        // slots per tile
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

// Tile lookup.  Slot tiles are numbered expert by expert, ceil(count/MT) per
// expert; each slot tile has n_tiles column tiles.  The grid is
// an upper bound on the tile count, so the numbering is made once the real
// count is known: the tiles are cut into 8 equal runs of consecutive numbers,
// run x going to the workgroups that the dispatcher places on XCD x (block
// numbers congruent to x mod 8).  The column tiles of one slot tile, and the
// next slot tile of the same expert, thus share an XCD's L2, and every XCD
// gets an equal share however many tiles there are.  Wave 0 scans the expert
// counts (up to 4 experts per lane); returns false for a workgroup without a
// tile.
__device__ bool find_tile(const int32_t* __restrict__ offsets, int E, int bid,
                          int n_tiles, int* s_res, int& e_out, int& base, int& cnt, int& ntile) {
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
        const int total = __shfl(incl, 63) * n_tiles;
        const int per_xcd = (total + 7) >> 3;
        const int lin = (bid & 7) * per_xcd + (bid >> 3);
        const bool have = (bid >> 3) < per_xcd && lin < total;
        const int tile = have ? lin / n_tiles : -1;
        int run = incl - tot;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (tile >= run && tile < run + t[q]) {
                const int e = lane * 4 + q, k = tile - run;
                s_res[0] = e;
                s_res[1] = offsets[e] + k * MT;
                s_res[2] = min(MT, c[q] - k * MT);
                s_res[3] = lin - tile * n_tiles;
            }
            run += t[q];
        }
        if (lane == 63 && !have) s_res[0] = -1;
    }
    __syncthreads();
    e_out = s_res[0];
    base = s_res[1];
    cnt = s_res[2];
    ntile = s_res[3];
    return e_out >= 0;
}

// MODE 0: gate/up.  act = permuted x [T][H], csum = -1.5 * block sums [T][H/32],
//         W = w_gate_up, rows_e = 2I, ncols = I; writes h (permuted) and its
//         block sums.
// MODE 1: down.     act = permuted h [N][I], csum [N][I/32], W = w_down,
//         rows_e = ncols = H; writes y_sorted.
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
// bytes apart, so three 16-byte loads that never cross the pair).  Each part
// of each stage is its own LDS array and the loop runs two iterations per trip
// with constant stage indices, so the compiler sees that the loads in flight
// do not touch what is being read (with one array for both stages it waited
// for every load before the reads).  The barrier is a bare s_barrier after an
// LDS-only wait: a memory-model fence would also drain the direct loads.
// Per wave and pair: MF/2 16-byte loads of activations (16 rows of one block
// each), one 4-byte load of block sums (64 rows of one block) and three
// 16-byte loads of weights (21 rows per instruction), in place of eight
// per-lane weight loads that each touched 16 rows.  A third weight stage (two
// pairs in flight) measured no faster for full tiles; tiles of at most 32
// slots, which have a quarter of the work per pair, run a three-stage ring.
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
    int nb, int rows_e, int ncols, int n_tiles, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_slots, int K, int E, uint16_t* __restrict__ h_out,
    float* __restrict__ hsum_out, float* __restrict__ y_out) {
    __shared__ __attribute__((aligned(16))) uint8_t a0[2 * MT * 64], a1[2 * MT * 64];
    __shared__ __attribute__((aligned(16))) float cc0[2 * MT], cc1[2 * MT];
    __shared__ __attribute__((aligned(16))) uint8_t w0[NT * 48], w1[NT * 48];
    // third stage of the light ring (tiles of at most 32 slots)
    __shared__ __attribute__((aligned(16))) uint8_t la2[2 * 32 * 64];
    __shared__ __attribute__((aligned(16))) float lc2[2 * 32];
    __shared__ __attribute__((aligned(16))) uint8_t w2[NT * 48];
    struct StageRef {
        uint8_t* a;
        float* c;
        uint8_t* w;
    };
    StageRef st0{a0, cc0, w0}, st1{a1, cc1, w1};
    __shared__ int s_res[4];

    int e, base, cnt, ntile;
    if (!find_tile(offsets, E, blockIdx.x, n_tiles, s_res, e, base, cnt, ntile)) return;
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

    // ---- this wave's weight rows ----
    // MODE 0: hidden columns c0 .. c0+31 (rows of gate, then the same rows of up)
    // MODE 1: output rows c0 .. c0+63
    const int c0 = MODE == 0 ? ntile * (NT / 2) + 32 * wave : ntile * NT + 64 * wave;
    int nfa;  // valid row fragments (whole wave for MODE 0)
    if (MODE == 0)
        nfa = c0 < ncols ? 4 : 0;
    else
        nfa = max(0, min(4, (ncols - c0) >> 4));
    // weight pieces: a row's 36 bytes of a pair as three 16-byte loads of its
    // bytes 0-15, 16-31 and 20-35 (never past the pair), 48 bytes per row in
    // LDS; lane piece i of a pair is q = 64 i + lane of the wave's 192 pieces,
    // row 16 nf + l16 = q / 3 of the wave, piece q % 3
    uint32_t woff[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int q = 64 * i + lane, r = q / 3;
        const int nf = r >> 4, rl = r & 15;
        int row;
        if (MODE == 0)
            row = min(c0 + (nf & 1) * 16 + rl, ncols - 1) + (nf >> 1) * ncols;
        else
            row = min(c0 + nf * 16 + rl, rows_e - 1);
        const int pc = q % 3;
        woff[i] = (uint32_t)row * rowbytes + (pc == 0 ? 0u : pc == 1 ? 16u : 20u);
    }
    // block sums: wave w loads block w >> 1 of tile rows 64 (w & 1) + lane
    int64_t cbyte0;  // byte offset in csum
    {
        const int r = 64 * (wave & 1) + lane;
        const int p = base + min(r, cnt - 1);
        const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
        cbyte0 = (arow * nb + (wave >> 1)) * 4;
    }
    // buffer resources (unbounded: every offset stays inside its buffer); the
    // fourth descriptor word selects 32-bit data, as untyped loads need
    constexpr int RSRC_W3 = 0x00020000;
    const __amdgpu_buffer_rsrc_t r_act = __builtin_amdgcn_make_buffer_rsrc((void*)act, 0, -1, RSRC_W3);
    const __amdgpu_buffer_rsrc_t r_cs = __builtin_amdgcn_make_buffer_rsrc((void*)csum, 0, -1, RSRC_W3);
    const __amdgpu_buffer_rsrc_t r_w = __builtin_amdgcn_make_buffer_rsrc((void*)We, 0, -1, RSRC_W3);

    const int mfa = min(8, (cnt + 15) >> 4);  // valid slot fragments
    const bool active = nfa > 0;

    // The main loop and epilogue for MF slot fragments (16 slots each).  A tile
    // of at most 32, 64 or 96 slots (an expert's last, partial tile, or a small
    // expert) runs with MF = 2, 4 or 6: a quarter, half or three quarters of
    // the activation loads, MFMAs and scale FMAs of a full tile.
    auto run = [&](auto mf_const) {
        constexpr int MF = decltype(mf_const)::value;
        constexpr int NA = MF / 2;  // activation loads per wave per pair
        constexpr bool LIGHT = MF == 2;
        constexpr int AROWS = LIGHT ? 32 : MT;  // rows per block in a stage
        f32x4 acc[MF][4];
#pragma unroll
        for (int i = 0; i < MF; ++i)
#pragma unroll
            for (int jn = 0; jn < 4; ++jn) acc[i][jn] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // activation loads: the WG's 2 MF instructions t = NA w + i cover block
        // t / MF, rows 16 (t % MF) .. +15; lane: row + (lane >> 2), LDS chunk
        // position lane & 3 holding the row's chunk (lane & 3) ^ ((row >> 2) & 3)
        int64_t abyte[NA];  // byte offsets in act
        int adst[NA];
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int t = NA * wave + i, blk = t / MF, rg = t % MF;
            const int r = 16 * rg + (lane >> 2);
            const int p = base + min(r, cnt - 1);
            const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
            const int chunk = (lane & 3) ^ ((r >> 2) & 3);
            abyte[i] = (arow * nb * 32 + blk * 32 + 8 * chunk) * 2;
            adst[i] = blk * AROWS * 64 + rg * 1024;
        }
        // block sums: a heavy stage takes block w >> 1 of rows 64 (w & 1) + lane
        // from wave w; a light stage its 2 x 32 sums (block lane >> 5, row
        // lane & 31) from every wave alike (the same bytes, so the four copies
        // agree)
        int64_t cbyte = cbyte0;
        int cdst = 64 * wave;
        if constexpr (LIGHT) {
            const int r = lane & 31;
            const int p = base + min(r, cnt - 1);
            const int64_t arow = MODE == 0 ? (int64_t)(sorted_slots[p] / K) : (int64_t)p;
            cbyte = (arow * nb + (lane >> 5)) * 4;
            cdst = 0;
        }
        // pair j: activations 128 bytes, block sums 8 bytes and weights 36 bytes
        // further on
        auto issue = [&](const StageRef& S, int j) {
            if constexpr (BUF) {
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(r_act, (lds_void_t*)(S.a + adst[i]), 16,
                                                             (int)abyte[i], 128 * j, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r_cs, (lds_void_t*)(S.c + cdst), 4,
                                                         (int)cbyte, 8 * j, 0, 0);
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        r_w, (lds_void_t*)(S.w + 64 * 48 * wave + 1024 * i), 16, (int)woff[i], 36 * j,
                        0, 0);
            } else {
                const uint8_t* act_b = reinterpret_cast<const uint8_t*>(act);
                const uint8_t* cs_b = reinterpret_cast<const uint8_t*>(csum);
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    __builtin_amdgcn_global_load_lds((glb_void_t*)(act_b + abyte[i] + 128 * j),
                                                     (lds_void_t*)(S.a + adst[i]), 16, 0, 0);
                __builtin_amdgcn_global_load_lds((glb_void_t*)(cs_b + cbyte + 8 * j),
                                                 (lds_void_t*)(S.c + cdst), 4, 0, 0);
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    __builtin_amdgcn_global_load_lds(
                        (glb_void_t*)(We + woff[i] + 36u * (uint32_t)j),
                        (lds_void_t*)(S.w + 64 * 48 * wave + 1024 * i), 16, 0, 0);
            }
        };
        const int swz = 16 * (g ^ ((l16 >> 2) & 3));  // this lane's chunk position in a row
        const int q1off = g < 3 ? 20 + 4 * g : 44;     // qs1 dword g in a row's 48 bytes
        // the nibble mask in a VGPR: each unpacking step is then a shift and a
        // v_and_or_b32 (a VOP3 operation takes no literal on gfx950)
        uint32_t nib_mask;
        asm volatile("v_mov_b32 %0, 0x00780078" : "=v"(nib_mask));
        auto compute = [&](const StageRef& S) {
            const uint8_t* WL = S.w + (wave * 64 + l16) * 48;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                // this block's weights: the scale and the lane's qs dword (block 0:
                // bytes 2 + 4g .. 5 + 4g of the pair, two dwords and an alignbyte;
                // block 1: bytes 20 + 4g .. 23 + 4g)
                float dv[4];
                u32x4 bq[4];
#pragma unroll
                for (int nf = 0; nf < 4; ++nf) {
                    const uint8_t* rp = WL + nf * 16 * 48;
                    if (blk == 0) {
                        const uint32_t lo = *(const uint32_t*)(rp + 4 * g);
                        const uint32_t hi = *(const uint32_t*)(rp + 4 * g + 4);
                        dv[nf] = f16_bits_to_f32(*(const uint16_t*)rp);
                        bq[nf] = dq_group(__builtin_amdgcn_alignbyte(hi, lo, 2), nib_mask);
                    } else {
                        dv[nf] = f16_bits_to_f32(*(const uint16_t*)(rp + 18));
                        bq[nf] = dq_group(*(const uint32_t*)(rp + q1off), nib_mask);
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
                        *(const u32x4*)(S.a + blk * AROWS * 64 + (mf * 16 + l16) * 64 + swz);
                    const f32x4 c = *(const f32x4*)&S.c[blk * AROWS + mf * 16 + 4 * g];
                    f32x4 t[4];
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf) t[nf] = mfma_bf16(a, bq[nf], c);
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[mf][nf][i] = fmaf(dv[nf], t[nf][i], acc[mf][nf][i]);
                }
            }
        };
        // One step per pair: issue the loads of a later pair (none past the
        // last), compute this pair, wait for this wave's loads of the next pair,
        // barrier.
        if constexpr (LIGHT) {
            // three stages (the third in arrays of its own): step j issues pair
            // j+2 into the stage pair j-1 used and waits for pair j+1 (issued a
            // step earlier)
            const StageRef st2{la2, lc2, w2};
            constexpr int OPS = NA + 4;  // direct loads per wave per pair
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
        if (MODE == 0) {
            // h = GELU(g) * u for hidden columns c0 .. c0+31: one Q4_0 block of the
            // down product's K, written in the MFMA order with its sum.  Each slot
            // fragment's 16 rows of 64 bytes go through a stage array of the wave's
            // own (rows 80 bytes apart, so the 4 lane groups' writes fall in
            // different banks) and leave as one 16-byte store per lane.
            const int I = ncols, nbh = I >> 5;
            const int hblk = c0 >> 5;
            constexpr int RB = 80;
            static_assert(MT * RB <= NT * 48 && NT * 48 <= 2 * MT * 64, "h staging fits");
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
                            *(uint16_t*)(R + r * RB + 2 * perm_pos(f * 16 + l16)) = hb;
                        }
                        // sum over the 16 lanes holding this row's columns
                        s += dpp_mov_f32<DPP_QUAD_XOR1>(s);
                        s += dpp_mov_f32<DPP_QUAD_XOR2>(s);
                        s += dpp_mov_f32<DPP_ROW_HALF_MIRROR>(s);
                        s += dpp_mov_f32<DPP_ROW_MIRROR>(s);
                        if (ok && l16 == 0) hsum_out[p * nbh + hblk] = -1.5f * s;
                    }
                    const int r = mf * 16 + (lane >> 2), ch = lane & 3;
                    const uint4 v = *(const uint4*)(R + r * RB + 16 * ch);
                    if (r < cnt) *(uint4*)(h_out + (int64_t)(base + r) * I + hblk * 32 + 8 * ch) = v;
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
            static_assert(32 * RS * 4 <= NT * 48 && NT * 48 <= 2 * MT * 64, "y staging fits");
            float* R = reinterpret_cast<float*>(wave == 0 ? a0 : wave == 1 ? a1 : wave == 2 ? w0 : w1);
            const int cq = lane & 15;
#pragma unroll
            for (int m2 = 0; m2 < MF; m2 += 2) {
                if (m2 < mfa) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int nf = 0; nf < 4; ++nf)
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
    if (cnt <= 32)
        run(std::integral_constant<int, 2>{});
    else if (cnt <= 64)
        run(std::integral_constant<int, 4>{});
    else if (cnt <= 96)
        run(std::integral_constant<int, 6>{});
    else
        run(std::integral_constant<int, 8>{});
}

// Activations -> MFMA block order, plus -1.5 * block sums.  Four lanes per
// 32-element block, one 16-byte quarter each (loads and stores of a wave are
// contiguous): output chunk c of a block holds elements 4c..4c+3 of quarter
// c >> 1 and elements 4c+16..4c+19 of quarter (c >> 1) + 2, which reach lane
// c through quad DPP moves.  The block sum is each lane's 8 values in order,
// then the quad's four partial sums.
__global__ __launch_bounds__(256) void ffn_mfma_prep(const uint16_t* __restrict__ x, int64_t nblocks,
                                                     uint16_t* __restrict__ xp,
                                                     float* __restrict__ xs) {
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
        reinterpret_cast<u32x4*>(xp)[q] = o;
        if (c == 0) xs[q >> 2] = -1.5f * s;
    }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t ffn_mfma_ws_bytes(int64_t T, int H, int I, int64_t N) {
    return align256((size_t)T * H * 2) + align256((size_t)T * (H / 32) * 4) +
           align256((size_t)N * I * 2) + align256((size_t)N * (I / 32) * 4);
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
    uint16_t* xp = (uint16_t*)p;
    p += align256((size_t)T * H * 2);
    float* xs = (float*)p;
    p += align256((size_t)T * (H / 32) * 4);
    uint16_t* hp = (uint16_t*)p;
    p += align256((size_t)N * I * 2);
    float* hs = (float*)p;

    const int64_t nblk = T * (H / 32);
    ffn_mfma_prep<<<(unsigned)((4 * nblk + 255) / 256), 256, 0, st>>>((const uint16_t*)x, nblk, xp, xs);

    // slot tiles: sum over experts of ceil(count / MT) <= N / MT + (experts hit);
    // the workgroups past the real count exit at once
    const int mtiles = N / MT + min(E, N);
    {
        const int n_tiles = (I + NT / 2 - 1) / (NT / 2);
        const int total = (mtiles * n_tiles + 7) / 8 * 8;
        if (buf_ok((size_t)T * H * 2))
            ffn_mfma<0, true><<<total, 256, 0, st>>>(xp, xs, w_gate_up, H / 32, 2 * I, I, n_tiles,
                                                     offsets, sorted_slots, K, E, hp, hs, nullptr);
        else
            ffn_mfma<0, false><<<total, 256, 0, st>>>(xp, xs, w_gate_up, H / 32, 2 * I, I, n_tiles,
                                                      offsets, sorted_slots, K, E, hp, hs, nullptr);
    }
    {
        const int n_tiles = (H + NT - 1) / NT;
        const int total = (mtiles * n_tiles + 7) / 8 * 8;
        if (buf_ok((size_t)N * I * 2))
            ffn_mfma<1, true><<<total, 256, 0, st>>>(hp, hs, w_down, I / 32, H, H, n_tiles, offsets,
                                                     sorted_slots, K, E, nullptr, nullptr, y_sorted);
        else
            ffn_mfma<1, false><<<total, 256, 0, st>>>(hp, hs, w_down, I / 32, H, H, n_tiles, offsets,
                                                      sorted_slots, K, E, nullptr, nullptr, y_sorted);
    }
    return hipGetLastError();
}

size_t linear_mfma_ws_bytes(int64_t T, int H) {
    return align256((size_t)T * H * 2) + align256((size_t)T * (H / 32) * 4);
}

hipError_t launch_linear_mfma(const void* x, int64_t T, int H, const uint8_t* W, int R,
                              const int32_t* offsets, const int32_t* slots, void* ws, float* y,
                              hipStream_t st) {
    uint16_t* xp = (uint16_t*)ws;
    float* xs = (float*)((uint8_t*)ws + align256((size_t)T * H * 2));
    const int64_t nblk = T * (H / 32);
    ffn_mfma_prep<<<(unsigned)((4 * nblk + 255) / 256), 256, 0, st>>>((const uint16_t*)x, nblk, xp, xs);
    const int N = (int)T, mtiles = N / MT + 1;
    const int n_tiles = (R + NT - 1) / NT;
    const int total = (mtiles * n_tiles + 7) / 8 * 8;
    if (buf_ok((size_t)T * H * 2))
        ffn_mfma<1, true><<<total, 256, 0, st>>>(xp, xs, W, H / 32, R, R, n_tiles, offsets, slots, 1,
                                                 1, nullptr, nullptr, y);
    else
        ffn_mfma<1, false><<<total, 256, 0, st>>>(xp, xs, W, H / 32, R, R, n_tiles, offsets, slots,
                                                  1, 1, nullptr, nullptr, y);
    return hipGetLastError();
}

}  // namespace moe
