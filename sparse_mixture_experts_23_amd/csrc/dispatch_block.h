// Count, scan and place of one block of T <= 256 tokens by one workgroup of 1024
// threads (E <= 1024) -- the same integer results as the multi-block dispatch
// kernels, with every block base slot 0 (no earlier block).
//
// Slot of path (t, e) = number of earlier tokens that selected e; ranks inside
// the block come from per-expert bit masks of the tokens (LDS atomic ORs, so
// order-independent), then L_e, min(L_e, C), the grouped-row offsets, the tile
// prefix, the overflow and the token statistics.
#pragma once

#include "common.h"

namespace {

// ids: [T, k] (global memory or LDS).  masks: 4 E uint64 and s_off: E int32 of
// LDS.  s_row (nullable, LDS): also receives row_of, complete when the function
// returns.  Every thread of the workgroup must call it (it holds workgroup
// barriers).
__device__ void dispatch_one_block(const int32_t* __restrict__ ids, int64_t T, int k, int E, int C,
                                   int32_t* __restrict__ load, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ stats, int32_t* __restrict__ tprefix, int tile_rows,
                                   int32_t* __restrict__ slot, int32_t* __restrict__ row_of,
                                   int32_t* __restrict__ src_token, unsigned long long* masks, int* s_off,
                                   int* s_row) {
    __shared__ int s_sum[16], s_over[16], s_max[16], s_tiles[16], s_drop[16], s_aff[16];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    for (int i = tid; i < 4 * E; i += 1024) masks[i] = 0ull;
    __syncthreads();
    if (tid < T) {
        for (int r = 0; r < k; ++r) {
            const int e = ids[tid * k + r];
            if ((unsigned)e < (unsigned)E) atomicOr(&masks[(tid / 64) * E + e], 1ull << (tid % 64));
        }
    }
    __syncthreads();
    // per expert: L_e, accepted, tiles; scans over e (thread e < E <= 1024)
    const int e = tid;
    int L = 0;
    if (e < E) {
#pragma unroll
        for (int w = 0; w < 4; ++w) L += __popcll(masks[w * E + e]);
    }
    const int acc = e < E ? min(L, C) : 0;
    const int over = e < E ? max(L - C, 0) : 0;
    const int tiles = tprefix ? (acc + tile_rows - 1) / tile_rows : 0;
    int incl = acc, tincl = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, MOE_WAVE);
        const int tv = __shfl_up(tincl, o, MOE_WAVE);
        if (lane >= o) {
            incl += v;
            tincl += tv;
        }
    }
    int ov = over, mx = L;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        ov += __shfl_xor(ov, o, MOE_WAVE);
        mx = max(mx, __shfl_xor(mx, o, MOE_WAVE));
    }
    if (lane == 63) {
        s_sum[wave] = incl;
        s_tiles[wave] = tincl;
    }
    if (lane == 0) {
        s_over[wave] = ov;
        s_max[wave] = mx;
    }
    __syncthreads();
    int before = 0, total = 0, otot = 0, mtot = 0, tbefore = 0, ttotal = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) {
            before += s_sum[w];
            tbefore += s_tiles[w];
        }
        total += s_sum[w];
        ttotal += s_tiles[w];
        otot += s_over[w];
        mtot = max(mtot, s_max[w]);
    }
    const int off = before + incl - acc;
    if (e < E) s_off[e] = off;
    __syncthreads();
    // place: token t = tid, rank = earlier tokens (lower lanes, lower waves) with e
    int dropped = 0, affected = 0;
    if (tid < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
        int nrej = 0;
        for (int r = 0; r < k; ++r) {
            const int ee = ids[tid * k + r];
            int c = -1, row = -1;
            if ((unsigned)ee < (unsigned)E) {
                int rank = __popcll(masks[wave * E + ee] & below);
                for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + ee]);
                if (rank < C) {
                    c = rank;
                    row = s_off[ee] + rank;
                    src_token[row] = tid;
                }
            }
            slot[tid * k + r] = c;
            row_of[tid * k + r] = row;
            if (s_row) s_row[tid * k + r] = row;
            nrej += c < 0;
        }
        dropped = nrej == k;
        affected = nrej > 0;
    }
    for (int o = 32; o >= 1; o >>= 1) {
        dropped += __shfl_xor(dropped, o, MOE_WAVE);
        affected += __shfl_xor(affected, o, MOE_WAVE);
    }
    if (lane == 0) {
        s_drop[wave] = dropped;
        s_aff[wave] = affected;
    }
    __syncthreads();
    // the per-expert results and the statistics are stored last, so no barrier above
    // waits for them
    if (e < E) {
        load[e] = L;
        offsets[e] = off;
        if (tprefix) tprefix[e] = tbefore + tincl - tiles;
    }
    if (tprefix && e < MOE_SCHED_WORDS) moe_sched_words(tprefix, E)[e] = 0ull;
    if (e == 0) {
        offsets[E] = total;
        if (tprefix) tprefix[E] = ttotal;
        int dsum = 0, asum = 0;
        for (int w = 0; w < 16; ++w) {
            dsum += s_drop[w];
            asum += s_aff[w];
        }
        stats[MOE_STAT_OVERFLOW] = otot;
        stats[MOE_STAT_ACCEPTED] = total;
        stats[MOE_STAT_MAX_LOAD] = mtot;
        stats[MOE_STAT_TOKENS_DROPPED] = dsum;
        stats[MOE_STAT_TOKENS_AFFECTED] = asum;
        for (int i = MOE_STAT_TOKENS_AFFECTED + 1; i < MOE_STAT_COUNT; ++i) stats[i] = 0;
    }
}

}  // namespace
