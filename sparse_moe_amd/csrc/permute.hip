// Token -> expert permutation: deterministic stable counting sort of the
// N = T*K (token, k) slots by expert, with per-expert offsets, gfx950.
//
// Within a tile of PERM_TILE slots (256 threads x 4 rounds), the stable rank of
// a slot among earlier slots of the same expert comes from a wave-level
// "match" of the 9-bit expert key (8 ballots) plus per-wave counts in LDS.
// One tile: a single workgroup finishes the sort.  Several tiles: per-tile
// counts -> one scan workgroup (prefix over tiles, then over experts) ->
// scatter.  No atomics; the result is unique.
#include "route_dev.h"

namespace moe {

// One tile: a single workgroup sorts every slot.
__global__ __launch_bounds__(64) void permute_one_wave(const int32_t* __restrict__ ids, int N, int E,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_slots,
                                                      int32_t* __restrict__ slot_pos) {
    permute_wave(ids, N, E, offsets, sorted_slots, slot_pos);
}

__global__ __launch_bounds__(256) void permute_single(const int32_t* __restrict__ ids, int N, int E,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_slots,
                                                      int32_t* __restrict__ slot_pos) {
    permute_block(ids, N, E, offsets, sorted_slots, slot_pos);
}

// Up to PERM_WIDE slots in one launch: one workgroup of 16 waves, 1024 slots
// per round.  Each (round, wave) pair counts its slots per expert (wave match)
// into its own row of a count table, so the rounds need no barriers between
// them; an exclusive prefix down each expert's column (rows in slot order)
// then gives every slot its stable rank, a scan over the experts the offsets.
constexpr int PERM_WIDE = 4096;

__global__ __launch_bounds__(1024) void permute_wide(const int32_t* __restrict__ ids, int N, int E,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_slots,
                                                     int32_t* __restrict__ slot_pos) {
    constexpr int RMAX = PERM_WIDE / 1024;
    __shared__ __align__(16) uint16_t cnt[RMAX * 16][MOE_MAX_E];
    __shared__ int seg[4][MOE_MAX_E];
    __shared__ int wsum[4];
    __shared__ int off[MOE_MAX_E];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rounds = (N + 1023) >> 10;
    const int R16 = rounds * 16;
    int ex[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const int s = r * 1024 + tid;
        const int v = ids[min(s, N - 1)];
        ex[r] = s < N ? v : -1;
    }
    uint4* z = reinterpret_cast<uint4*>(&cnt[0][0]);
    for (int i = tid; i < R16 * MOE_MAX_E / 8; i += 1024) z[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    int rw[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        rw[r] = 0;
        if (r < rounds) {
            const uint32_t key = ex[r] >= 0 ? (uint32_t)ex[r] : 256u;
            const uint64_t m = match_key9(key);
            rw[r] = __popcll(m & lanemask_lt());
            if (ex[r] >= 0 && rw[r] == 0) cnt[r * 16 + wave][ex[r]] = (uint16_t)__popcll(m);
        }
    }
    __syncthreads();
    // column prefix: four threads per expert, each over a quarter of the rows
    const int col = tid & (MOE_MAX_E - 1), sg = tid >> 8, per = R16 >> 2;
    int sum = 0;
    for (int i = 0; i < per; ++i) sum += cnt[sg * per + i][col];
    seg[sg][col] = sum;
    __syncthreads();
    int base = 0;
    for (int q = 0; q < sg; ++q) base += seg[q][col];
    for (int i = 0; i < per; ++i) {
        const int c = cnt[sg * per + i][col];
        cnt[sg * per + i][col] = (uint16_t)base;
        base += c;
    }
    // exclusive scan of the expert totals by the first four waves
    int incl = 0, tot = 0;
    if (tid < MOE_MAX_E) {
        tot = col < E ? seg[0][col] + seg[1][col] + seg[2][col] + seg[3][col] : 0;
        incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < MOE_MAX_E) {
        for (int q = 0; q < wave; ++q) incl += wsum[q];
        if (col < E) {
            off[col] = incl - tot;
            offsets[col] = incl - tot;
        }
        if (col == E - 1) offsets[E] = incl;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const int s = r * 1024 + tid;
        if (ex[r] >= 0) {
            const int pos = off[ex[r]] + cnt[r * 16 + wave][ex[r]] + rw[r];
            sorted_slots[pos] = s;
            slot_pos[s] = pos;
        }
    }
}

// Several tiles: per-tile stable ranks and per-expert tile counts.
__global__ __launch_bounds__(256) void permute_tiles(const int32_t* __restrict__ ids, int N, int E,
                                                     int32_t* __restrict__ tile_counts,
                                                     int32_t* __restrict__ local_rank) {
    __shared__ int run[MOE_MAX_E];
    __shared__ int wcnt[4][MOE_MAX_E];
    const int tid = threadIdx.x, wave = tid >> 6;
    run[tid] = 0;  // blockDim == MOE_MAX_E
    const int base = blockIdx.x * PERM_TILE;
#pragma unroll
    for (int r = 0; r < PERM_TILE / 256; ++r) {
        const int s = base + r * 256 + tid;
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
        if (valid) {
            int rk = rw + run[e];
            for (int w = 0; w < wave; ++w) rk += wcnt[w][e];
            local_rank[s] = rk;
        }
        __syncthreads();
        run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        __syncthreads();
    }
    if (tid < E) tile_counts[(int64_t)blockIdx.x * E + tid] = run[tid];
}

// Scatter, with the scan folded in: every workgroup sums the per-expert tile
// counts itself (its tile's base is the sum over the earlier tiles; the expert
// offsets, a scan of the totals, are the same in every workgroup and the first
// one stores them), which saves the launch of a one-workgroup scan.
__global__ __launch_bounds__(256) void permute_scatter(const int32_t* __restrict__ ids, int N, int E,
                                                       int ntiles,
                                                       const int32_t* __restrict__ tile_counts,
                                                       const int32_t* __restrict__ local_rank,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_slots,
                                                       int32_t* __restrict__ slot_pos) {
    __shared__ int tb[MOE_MAX_E];
    __shared__ int tot[256];
    __shared__ int tmp[256];
    __shared__ int off[MOE_MAX_E + 1];
    const int e = threadIdx.x;
    const int me = blockIdx.x;
    int before = 0, all = 0;
    if (e < E) {
        int tile = 0;
        for (; tile + 8 <= ntiles; tile += 8) {
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = tile_counts[(int64_t)(tile + i) * E + e];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                before += tile + i < me ? c[i] : 0;
                all += c[i];
            }
        }
        for (; tile < ntiles; ++tile) {
            const int c = tile_counts[(int64_t)tile * E + e];
            before += tile < me ? c : 0;
            all += c;
        }
        tb[e] = before;
    }
    tot[e] = all;
    __syncthreads();
    block_exclusive_scan256(tot, E, tmp, me == 0 ? offsets : nullptr, off);
    const int base = me * PERM_TILE;
#pragma unroll
    for (int r = 0; r < PERM_TILE / 256; ++r) {
        const int s = base + r * 256 + threadIdx.x;
        if (s < N) {
            const int ex = ids[s];
            const int pos = off[ex] + tb[ex] + local_rank[s];
            sorted_slots[pos] = s;
            slot_pos[s] = pos;
        }
    }
}

size_t permute_ws_bytes(int64_t N, int E) {
    if (N <= PERM_WIDE) return 0;
    const int64_t ntiles = (N + PERM_TILE - 1) / PERM_TILE;
    return (size_t)(ntiles * E + N) * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* ids, int N, int E, int32_t* offsets, int32_t* sorted_slots,
                          int32_t* slot_pos, void* ws, hipStream_t st) {
    if (N <= PERM_WAVE) {
        permute_one_wave<<<1, 64, 0, st>>>(ids, N, E, offsets, sorted_slots, slot_pos);
        return hipGetLastError();
    }
    if (N <= PERM_TILE) {
        permute_single<<<1, 256, 0, st>>>(ids, N, E, offsets, sorted_slots, slot_pos);
        return hipGetLastError();
    }
    if (N <= PERM_WIDE) {
        permute_wide<<<1, 1024, 0, st>>>(ids, N, E, offsets, sorted_slots, slot_pos);
        return hipGetLastError();
    }
    const int ntiles = (N + PERM_TILE - 1) / PERM_TILE;
    int32_t* tile_counts = (int32_t*)ws;
    int32_t* local_rank = tile_counts + (int64_t)ntiles * E;
    permute_tiles<<<ntiles, 256, 0, st>>>(ids, N, E, tile_counts, local_rank);
    permute_scatter<<<ntiles, 256, 0, st>>>(ids, N, E, ntiles, tile_counts, local_rank, offsets,
                                            sorted_slots, slot_pos);
    return hipGetLastError();
}

}  // namespace moe
