// Capacity-limited dispatch: slots in token order, grouped row map, row gather,
// load statistics.
//
// Definition ("LLM from scratch" ch. 36 Algorithm 36.1 acceptance step, §36.3):
// per-expert counters start at 0; token by token, each selected path takes the
// next slot of its expert if fewer than C slots are used, otherwise it is
// rejected.  Because a token selects each expert at most once, the slot of path
// (t, e) equals the number of earlier tokens that selected e -- an exclusive
// prefix count in token order -- so the serial definition is computed here in
// parallel, exactly:
//   count : per 256-token block, the tokens selecting each expert
//   scan  : per expert, exclusive prefix over blocks; L_e, min(L_e, C),
//           grouped-row offsets, overflow O ("The real cost of sparse expert
//           models", equations for C_e and O), max load
//   place : rank inside the block = popcount of a per-expert bit mask of the
//           earlier lanes (built with order-independent LDS atomic ORs), so
//           the result never depends on thread timing
//   gather: x_perm[row] = x[token], one wave per token, 16-byte vector copies.
// Where the rows are copied and no router table exists, scan and place run
// inside the gather's workgroups (dispatch_place_gather_kernel), on ranks the
// count kernel leaves in `slot`.
#include "common.h"
#include "dispatch_block.h"

namespace {

constexpr int DB_TOK = MOE_DISPATCH_BLOCK;   // tokens per count/place workgroup (4 waves x 64)

__device__ __forceinline__ void build_masks(unsigned long long* masks, const int32_t* __restrict__ ids, int64_t T,
                                            int k, int E) {
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    for (int i = tid; i < 4 * E; i += DB_TOK) masks[i] = 0ull;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * DB_TOK + tid;
    if (t < T) {
        for (int r = 0; r < k; ++r) {
            const int e = ids[t * k + r];
            if ((unsigned)e < (unsigned)E) atomicOr(&masks[wave * E + e], 1ull << lane);
        }
    }
    __syncthreads();
}

// acc_stats (nullable): the two statistics the placement accumulates with atomics,
// cleared here (block 0) for the placement kernels.
// rank (nullable): also each path's rank among the block's paths to its expert,
// in token order (0 for an id out of range), rank[t k + r].
__global__ __launch_bounds__(DB_TOK) void dispatch_count_kernel(const int32_t* __restrict__ ids, int64_t T, int k,
                                                                int E, int32_t* __restrict__ hist,
                                                                int32_t* __restrict__ acc_stats,
                                                                int32_t* __restrict__ rank) {
    extern __shared__ unsigned long long masks[];
    if (acc_stats && blockIdx.x == 0 && threadIdx.x < 2) acc_stats[threadIdx.x] = 0;
    build_masks(masks, ids, T, k, E);
    for (int e = threadIdx.x; e < E; e += DB_TOK) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) c += __popcll(masks[w * E + e]);
        hist[(int64_t)blockIdx.x * E + e] = c;
    }
    const int64_t t = (int64_t)blockIdx.x * DB_TOK + threadIdx.x;
    if (rank && t < T) {
        const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int r = 0; r < k; ++r) {
            const int ee = ids[t * k + r];
            int n = 0;
            if ((unsigned)ee < (unsigned)E) {
                n = __popcll(masks[wave * E + ee] & below);
                for (int w = 0; w < wave; ++w) n += __popcll(masks[w * E + ee]);
            }
            rank[t * k + r] = n;
        }
    }
}

// Scans over the experts for one 256-thread workgroup: thread e < E (E <= 256)
// brings L (= L_e) and base (the paths to e in the token blocks before this
// workgroup's); on return (after a barrier) s_off[e] holds expert e's first
// grouped row and s_base[e] its base.  Workgroup 0 also writes load, offsets,
// the tile prefix (tprefix nullable; tprefix[e] = tiles of the experts before e,
// rows per tile tile_rows) and the load statistics, and clears the other
// statistics but the two token counts.
__device__ __forceinline__ void expert_scan(int L, int base, int E, int C, int* s_off, int* s_base,
                                            int32_t* __restrict__ load, int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ stats, int32_t* __restrict__ tprefix,
                                            int tile_rows) {
    __shared__ int s_sum[4], s_tiles[4], s_over[4], s_max[4];
    const int e = threadIdx.x, wave = e / 64, lane = e % 64;
    const int acc = e < E ? min(L, C) : 0;
    const int over = e < E ? max(L - C, 0) : 0;
    const int tiles = tprefix ? (acc + tile_rows - 1) / tile_rows : 0;
    int incl = acc, tincl = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int sv = __shfl_up(incl, o, MOE_WAVE);
        const int tv = __shfl_up(tincl, o, MOE_WAVE);
        if (lane >= o) {
            incl += sv;
            tincl += tv;
        }
    }
    int ov = over, mx = e < E ? L : 0;
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
#pragma unroll
    for (int w = 0; w < 4; ++w) {
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
    if (e < E) {
        s_off[e] = off;
        s_base[e] = base;
    }
    if (blockIdx.x == 0) {
        if (e < E) {
            load[e] = L;
            offsets[e] = off;
            if (tprefix) tprefix[e] = tbefore + tincl - tiles;
        }
        if (tprefix && e < MOE_SCHED_WORDS) moe_sched_words(tprefix, E)[e] = 0ull;
        if (e == 0) {
            offsets[E] = total;
            if (tprefix) tprefix[E] = ttotal;
            stats[MOE_STAT_OVERFLOW] = otot;
            stats[MOE_STAT_ACCEPTED] = total;
            stats[MOE_STAT_MAX_LOAD] = mtot;
            for (int i = MOE_STAT_TOKENS_AFFECTED + 1; i < MOE_STAT_COUNT; ++i) stats[i] = 0;
        }
    }
    __syncthreads();
}

// One workgroup of 1024 threads (E <= 1024): thread e scans expert e over blocks.
// tprefix (nullable): also writes the grouped GEMMs' tile prefix,
// tprefix[e] = sum_{e' < e} ceil(accepted(e') / tile_rows), tprefix[E] = total.
// roff (nullable): also the exclusive prefix of the requested loads, roff[e] and
// roff[E] = T k (positions of each expert's requests, acceptance by gate weight).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ hist, int NB, int E, int C,
                                                             int32_t* __restrict__ load, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ stats, int32_t* __restrict__ tprefix,
                                                             int tile_rows, int32_t* __restrict__ roff) {
    __shared__ int s_sum[16], s_over[16], s_max[16], s_tiles[16], s_req[16];
    const int e = threadIdx.x, wave = e / 64, lane = e % 64;
    int L = 0;
    if (e < E) {
        for (int b = 0; b < NB; ++b) {
            const int h = hist[(int64_t)b * E + e];
            hist[(int64_t)b * E + e] = L;   // becomes the block's base slot for expert e
            L += h;
        }
        load[e] = L;
    }
    const int acc = e < E ? min(L, C) : 0;
    const int over = e < E ? max(L - C, 0) : 0;
    const int tiles = tprefix ? (acc + tile_rows - 1) / tile_rows : 0;
    // inclusive wave scans of acc, of the tile counts and of the requests
    int incl = acc, tincl = tiles, rincl = L;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, MOE_WAVE);
        const int tv = __shfl_up(tincl, o, MOE_WAVE);
        const int rv = __shfl_up(rincl, o, MOE_WAVE);
        if (lane >= o) {
            incl += v;
            tincl += tv;
            rincl += rv;
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
        s_req[wave] = rincl;
    }
    if (lane == 0) {
        s_over[wave] = ov;
        s_max[wave] = mx;
    }
    __syncthreads();
    int before = 0, total = 0, otot = 0, mtot = 0, tbefore = 0, ttotal = 0, rbefore = 0, rtotal = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) {
            before += s_sum[w];
            tbefore += s_tiles[w];
            rbefore += s_req[w];
        }
        total += s_sum[w];
        ttotal += s_tiles[w];
        rtotal += s_req[w];
        otot += s_over[w];
        mtot = max(mtot, s_max[w]);
    }
    if (e < E) offsets[e] = before + incl - acc;
    if (tprefix && e < E) tprefix[e] = tbefore + tincl - tiles;
    if (tprefix && e == 0) tprefix[E] = ttotal;
    if (tprefix && e < MOE_SCHED_WORDS) moe_sched_words(tprefix, E)[e] = 0ull;
    if (roff && e < E) roff[e] = rbefore + rincl - (e < E ? L : 0);
    if (roff && e == 0) roff[E] = rtotal;
    if (e == 0) {
        offsets[E] = total;
        stats[MOE_STAT_OVERFLOW] = otot;
        stats[MOE_STAT_ACCEPTED] = total;
        stats[MOE_STAT_MAX_LOAD] = mtot;
        for (int i = MOE_STAT_TOKENS_DROPPED; i < MOE_STAT_COUNT; ++i) stats[i] = 0;
    }
}

__global__ __launch_bounds__(DB_TOK) void dispatch_place_kernel(const int32_t* __restrict__ ids, int64_t T, int k,
                                                                int E, int C, const int32_t* __restrict__ base,
                                                                const int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ slot, int32_t* __restrict__ row_of,
                                                                int32_t* __restrict__ src_token,
                                                                int32_t* __restrict__ stats) {
    extern __shared__ unsigned long long masks[];
    __shared__ int s_drop[4], s_aff[4];
    build_masks(masks, ids, T, k, E);
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int64_t t = (int64_t)blockIdx.x * DB_TOK + tid;
    int dropped = 0, affected = 0;
    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
        int nrej = 0;
        for (int r = 0; r < k; ++r) {
            const int e = ids[t * k + r];
            int c = -1, row = -1;
            if ((unsigned)e < (unsigned)E) {
                int rank = __popcll(masks[wave * E + e] & below);
                for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + e]);
                const int cand = base[(int64_t)blockIdx.x * E + e] + rank;
                if (cand < C) {
                    c = cand;
                    row = offsets[e] + cand;
                    src_token[row] = (int32_t)t;
                }
            }
            slot[t * k + r] = c;
            row_of[t * k + r] = row;
            nrej += c < 0;
        }
        dropped = nrej == k;
        affected = nrej > 0;
    }
    // workgroup sums, then one integer atomic add each (order-independent)
    for (int o = 32; o >= 1; o >>= 1) {
        dropped += __shfl_xor(dropped, o, MOE_WAVE);
        affected += __shfl_xor(affected, o, MOE_WAVE);
    }
    if (lane == 0) {
        s_drop[wave] = dropped;
        s_aff[wave] = affected;
    }
    __syncthreads();
    if (tid == 0) {
        const int dsum = s_drop[0] + s_drop[1] + s_drop[2] + s_drop[3];
        const int asum = s_aff[0] + s_aff[1] + s_aff[2] + s_aff[3];
        if (dsum) atomicAdd(&stats[MOE_STAT_TOKENS_DROPPED], dsum);
        if (asum) atomicAdd(&stats[MOE_STAT_TOKENS_AFFECTED], asum);
    }
}

// Scan + place for small count tables (NR * E <= 4096, E <= 256): every block's
// workgroup loads the whole count table into LDS and derives from it the totals
// L_e, its own base slots and the grouped-row offsets (the same integer results
// as dispatch_scan_kernel), then places its tokens as dispatch_place_kernel does
// -- one launch instead of two.  The table has NR rows, `sub` per 256-token
// block: one row per block (the count kernel) or one per router workgroup of
// MOE_ROUTE_TOK tokens; a block's base is the sum of the rows before its first.  Block 0 also
// writes load, offsets, the tile prefix and the statistics; the token statistics
// are accumulated with atomics into counters the kernel that filled the table has
// cleared.  Dynamic LDS: masks (4 E uint64), then s_base[E], s_off[E],
// s_hist[NR E] int32.
constexpr int SCAN_INLINE_MAX = 4096;
__global__ __launch_bounds__(DB_TOK) void dispatch_place_scan_kernel(
    const int32_t* __restrict__ ids, int64_t T, int k, int E, int C, const int32_t* __restrict__ hist, int NR, int sub,
    int32_t* __restrict__ load, int32_t* __restrict__ offsets, int32_t* __restrict__ slot,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_token, int32_t* __restrict__ stats,
    int32_t* __restrict__ tprefix, int tile_rows, int32_t* __restrict__ status, int32_t* __restrict__ route_flag) {
    extern __shared__ unsigned long long masks[];
    int* s_base = reinterpret_cast<int*>(masks + 4 * E);
    // the router's non-finite flag -> the status word (the router launch has ended)
    if (status && blockIdx.x == 0 && threadIdx.x == 0)
        *status = atomicExch(route_flag, 0) ? MOE_ERR_NONFINITE_LOGIT : MOE_OK;
    int* s_off = s_base + E;
    int* s_hist = s_off + E;
    __shared__ int s_drop[4], s_aff[4];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int n = NR * E;
    {   // the table: up to 16 loads per thread, all in flight together
        int v[SCAN_INLINE_MAX / DB_TOK];
#pragma unroll
        for (int u = 0; u < SCAN_INLINE_MAX / DB_TOK; ++u) v[u] = hist[min(tid + DB_TOK * u, n - 1)];
#pragma unroll
        for (int u = 0; u < SCAN_INLINE_MAX / DB_TOK; ++u)
            if (tid + DB_TOK * u < n) s_hist[tid + DB_TOK * u] = v[u];
    }
    build_masks(masks, ids, T, k, E);   // its barriers also publish s_hist
    // thread e < E <= 256: L_e and this block's base, then the scans over e
    const int e = tid;
    int L = 0, base = 0;
    if (e < E) {
        const int first = (int)blockIdx.x * sub;   // this block's first row
        for (int b = 0; b < NR; ++b) {
            const int h = s_hist[b * E + e];
            base += b < first ? h : 0;
            L += h;
        }
    }
    expert_scan(L, base, E, C, s_off, s_base, load, offsets, stats, tprefix, tile_rows);
    // place: as dispatch_place_kernel, with this block's bases from LDS
    const int64_t t = (int64_t)blockIdx.x * DB_TOK + tid;
    int dropped = 0, affected = 0;
    if (t < T) {
        const unsigned long long below = (1ull << lane) - 1ull;
        int nrej = 0;
        for (int r = 0; r < k; ++r) {
            const int ee = ids[t * k + r];
            int c = -1, row = -1;
            if ((unsigned)ee < (unsigned)E) {
                int rank = __popcll(masks[wave * E + ee] & below);
                for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + ee]);
                const int cand = s_base[ee] + rank;
                if (cand < C) {
                    c = cand;
                    row = s_off[ee] + cand;
                    src_token[row] = (int32_t)t;
                }
            }
            slot[t * k + r] = c;
            row_of[t * k + r] = row;
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
    if (tid == 0) {
        const int dsum = s_drop[0] + s_drop[1] + s_drop[2] + s_drop[3];
        const int asum = s_aff[0] + s_aff[1] + s_aff[2] + s_aff[3];
        if (dsum) atomicAdd(&stats[MOE_STAT_TOKENS_DROPPED], dsum);
        if (asum) atomicAdd(&stats[MOE_STAT_TOKENS_AFFECTED], asum);
    }
}

// T <= 256 (one token block): count, scan and place in one workgroup of 1024
// threads.  masks: 4 E uint64 of dynamic LDS, then s_off[E] int32.
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ ids, int64_t T, int k,
                                                              int E, int C, int32_t* __restrict__ load,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ stats,
                                                              int32_t* __restrict__ tprefix, int tile_rows,
                                                              int32_t* __restrict__ slot,
                                                              int32_t* __restrict__ row_of,
                                                              int32_t* __restrict__ src_token) {
    extern __shared__ unsigned long long masks[];
    int* s_off = reinterpret_cast<int*>(masks + 4 * E);
    dispatch_one_block(ids, T, k, E, C, load, offsets, stats, tprefix, tile_rows, slot, row_of, src_token, masks,
                       s_off, nullptr);
}

// ---------------------------------------------------------------------------
// Overflow variant: acceptance by gate weight ("LLM from scratch" ch. 36 §36.3,
// acceptance rules).  An expert over capacity keeps its C requests of largest
// routing weight, equal weights in token order; the accepted rows keep token
// order.  Priority key of request (t, e) = (bits of its fp32 weight << 32) |
// ~t: the weights are positive, so their bit patterns order like the values,
// and a larger key is a higher priority; within an expert keys are unique.
// ---------------------------------------------------------------------------

// Per 256-token block: every request (t, r) goes to position roff[e] + (its
// first-come position among e's requests) of the request lists (key, path id);
// paths with an invalid id get slot / row -1 here.
__global__ __launch_bounds__(DB_TOK) void dispatch_requests_kernel(const int32_t* __restrict__ ids,
                                                                   const float* __restrict__ w, int64_t T, int k,
                                                                   int E, const int32_t* __restrict__ base,
                                                                   const int32_t* __restrict__ roff,
                                                                   unsigned long long* __restrict__ req_key,
                                                                   int32_t* __restrict__ req_path,
                                                                   int32_t* __restrict__ slot,
                                                                   int32_t* __restrict__ row_of) {
    extern __shared__ unsigned long long masks[];
    build_masks(masks, ids, T, k, E);
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int64_t t = (int64_t)blockIdx.x * DB_TOK + tid;
    if (t >= T) return;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int r = 0; r < k; ++r) {
        const int e = ids[t * k + r];
        if ((unsigned)e >= (unsigned)E) {
            slot[t * k + r] = -1;
            row_of[t * k + r] = -1;
            continue;
        }
        int rank = __popcll(masks[wave * E + e] & below);
        for (int q = 0; q < wave; ++q) rank += __popcll(masks[q * E + e]);
        const int64_t pos = (int64_t)roff[e] + base[(int64_t)blockIdx.x * E + e] + rank;
        req_key[pos] = ((unsigned long long)__float_as_uint(w[t * k + r]) << 32) |
                       (unsigned long long)(0xffffffffu - (uint32_t)t);
        req_path[pos] = (int32_t)(t * k + r);
    }
}

// Workgroup e: the C-th largest key of expert e's requests (radix selection, 8
// bits a pass from the top: each pass counts the candidates' next digit with LDS
// atomics and keeps the digit where the count from the top reaches C); 0 (every
// key passes) when the expert is not over capacity.
__global__ __launch_bounds__(1024) void dispatch_threshold_kernel(const int32_t* __restrict__ load,
                                                                  const int32_t* __restrict__ roff, int C,
                                                                  const unsigned long long* __restrict__ req_key,
                                                                  unsigned long long* __restrict__ thresh) {
    __shared__ int hist[256], wsum[4];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_need, s_need_next;
    const int e = blockIdx.x, tid = threadIdx.x;
    const int L = load[e];
    if (L <= C) {
        if (tid == 0) thresh[e] = 0ull;
        return;
    }
    const unsigned long long* key = req_key + roff[e];
    if (tid == 0) {
        s_prefix = 0ull;
        s_need = C;
    }
    unsigned long long mask = 0ull;
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += 1024) hist[i] = 0;
        __syncthreads();
        const unsigned long long prefix = s_prefix;
        for (int i = tid; i < L; i += 1024) {
            const unsigned long long kk = key[i];
            if ((kk & mask) == prefix) atomicAdd(&hist[(int)((kk >> shift) & 0xffull)], 1);
        }
        __syncthreads();
        // counts from the largest digit down: thread i < 256 takes digit 255 - i;
        // the digit where the running count first reaches `need` is chosen
        const int need = s_need;
        const int lane = tid % 64, wave = tid / 64;
        int v = 0, incl = 0;
        if (tid < 256) {   // waves 0..3, whole waves
            v = hist[255 - tid];
            incl = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_up(incl, o, MOE_WAVE);
                if (lane >= o) incl += u;
            }
            if (lane == 63) wsum[wave] = incl;
        }
        __syncthreads();   // every wave of the workgroup
        if (tid < 256) {
            for (int q = 0; q < wave; ++q) incl += wsum[q];
            const int excl = incl - v;
            if (excl < need && incl >= need) {
                s_need_next = need - excl;
                s_prefix = prefix | ((unsigned long long)(255 - tid) << shift);
            }
        }
        mask |= 0xffull << shift;
        __syncthreads();
        if (tid == 0) s_need = s_need_next;
        __syncthreads();
    }
    if (tid == 0) thresh[e] = s_prefix;
}

// Workgroup e: walks expert e's requests in first-come order; those with key >=
// thresh[e] are accepted and numbered in that (token) order.
__global__ __launch_bounds__(1024) void dispatch_assign_kernel(const int32_t* __restrict__ load,
                                                               const int32_t* __restrict__ roff,
                                                               const int32_t* __restrict__ offsets, int k,
                                                               const unsigned long long* __restrict__ req_key,
                                                               const int32_t* __restrict__ req_path,
                                                               const unsigned long long* __restrict__ thresh,
                                                               int32_t* __restrict__ slot,
                                                               int32_t* __restrict__ row_of,
                                                               int32_t* __restrict__ src_token) {
    __shared__ int w_cnt[16];
    const int e = blockIdx.x, tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int L = load[e], base = roff[e], off = offsets[e];
    const unsigned long long th = thresh[e];
    int running = 0;
    for (int i0 = 0; i0 < L; i0 += 1024) {
        const int i = i0 + tid;
        const bool in = i < L;
        const bool acc = in && req_key[base + i] >= th;
        const unsigned long long bal = __ballot(acc);
        const int before_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) w_cnt[wave] = __popcll(bal);
        __syncthreads();
        int before = running + before_in_wave, chunk = 0;
        for (int q = 0; q < 16; ++q) {
            if (q < wave) before += w_cnt[q];
            chunk += w_cnt[q];
        }
        if (in) {
            const int path = req_path[base + i];
            if (acc) {
                slot[path] = before;
                row_of[path] = off + before;
                src_token[off + before] = path / k;
            } else {
                slot[path] = -1;
                row_of[path] = -1;
            }
        }
        running += chunk;
        __syncthreads();
    }
}

// Tokens with some / all paths rejected, per 256-token block (one atomic add each).
__global__ __launch_bounds__(DB_TOK) void dispatch_token_stats_kernel(const int32_t* __restrict__ row_of, int64_t T,
                                                                      int k, int32_t* __restrict__ stats) {
    __shared__ int s_drop[4], s_aff[4];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int64_t t = (int64_t)blockIdx.x * DB_TOK + tid;
    int dropped = 0, affected = 0;
    if (t < T) {
        int nrej = 0;
        for (int r = 0; r < k; ++r) nrej += row_of[t * k + r] < 0;
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
    if (tid == 0) {
        const int dsum = s_drop[0] + s_drop[1] + s_drop[2] + s_drop[3];
        const int asum = s_aff[0] + s_aff[1] + s_aff[2] + s_aff[3];
        if (dsum) atomicAdd(&stats[MOE_STAT_TOKENS_DROPPED], dsum);
        if (asum) atomicAdd(&stats[MOE_STAT_TOKENS_AFFECTED], asum);
    }
}

// x_perm[row] = x[t] for every accepted path of token t; one wave per token.
template <typename V>
__global__ __launch_bounds__(256) void dispatch_gather_kernel(const V* __restrict__ x, int64_t T, int k,
                                                              int64_t vec_per_row, const int32_t* __restrict__ row_of,
                                                              V* __restrict__ x_perm) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int myrow = lane < k ? row_of[t * k + lane] : -1;
    const V* src = x + t * vec_per_row;
    // uniform trip count: every lane stays active around lane_value
    for (int64_t c0 = 0; c0 < vec_per_row; c0 += 64) {
        const int64_t c = c0 + lane;
        const bool ok = c < vec_per_row;
        V v;
        if (ok) v = src[c];
        for (int r = 0; r < k; ++r) {
            const int row = lane_value(myrow, r);
            if (row >= 0 && ok) x_perm[(int64_t)row * vec_per_row + c] = v;
        }
    }
}

// The standalone dispatch's placement, fused into its row gather.  The count
// kernel has written the per-block table hist[NB][E] and, into `slot`, each
// path's rank inside its 256-token block.  Every workgroup (4 tokens, one wave
// each) scans the table for its block's bases and the grouped offsets, places
// its tokens' paths (slot, row_of, src_token, as the separate placement would)
// and copies their rows, whose first NPF 64-lane chunks are already in flight
// while the table is scanned: the placement rides on the copy instead of taking
// a launch of its own.  Workgroup 0 writes load, offsets, the tile prefix and
// the load statistics; the two token statistics are left to
// dispatch_token_stats_kernel (one atomic add per 256 tokens instead of one per
// workgroup here, which serialise on their two words).  Dynamic LDS: s_base[E],
// s_off[E], s_hist[NB E] int32.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16-byte chunks (kept in registers)
template <typename V, int NPF>
__global__ __launch_bounds__(256) void dispatch_place_gather_kernel(
    const V* __restrict__ x, const int32_t* __restrict__ ids, int64_t T, int k, int E, int C,
    const int32_t* __restrict__ hist, int NB, int32_t* __restrict__ load, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot, int32_t* __restrict__ row_of, int32_t* __restrict__ src_token,
    int32_t* __restrict__ stats, int32_t* __restrict__ tprefix, int tile_rows, int64_t vec_per_row,
    V* __restrict__ x_perm) {
    extern __shared__ int s_base[];
    int* s_off = s_base + E;
    int* s_hist = s_off + E;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    const bool live = t < T;
    const V* src = x + (live ? t : 0) * vec_per_row;
    V v[NPF];   // unconditional loads (clamped into the row), all in flight together
#pragma unroll
    for (int u = 0; u < NPF; ++u) v[u] = src[min((int64_t)u * 64 + lane, vec_per_row - 1)];
    // lane r < k: path r's expert and rank (loaded with the row, used after the scan)
    const int64_t pr = (live ? t : 0) * k + min(lane, k - 1);
    const int my_e = ids[pr], my_rank = slot[pr];
    {   // the table into LDS: up to 16 loads per thread, all in flight together
        const int n = NB * E;
        int h[SCAN_INLINE_MAX / 256];
#pragma unroll
        for (int u = 0; u < SCAN_INLINE_MAX / 256; ++u) h[u] = hist[min(tid + 256 * u, n - 1)];
#pragma unroll
        for (int u = 0; u < SCAN_INLINE_MAX / 256; ++u)
            if (tid + 256 * u < n) s_hist[tid + 256 * u] = h[u];
    }
    __syncthreads();
    // thread e < E: L_e over all blocks, base = paths to e in the blocks before this one
    const int blk = (int)((int64_t)blockIdx.x * 4 / DB_TOK);
    int L = 0, base = 0;
    if (tid < E) {
        for (int b = 0; b < NB; ++b) {
            const int h = s_hist[b * E + tid];
            base += b < blk ? h : 0;
            L += h;
        }
    }
    expert_scan(L, base, E, C, s_off, s_base, load, offsets, stats, tprefix, tile_rows);
    // lane r < k places path r of this wave's token
    int myrow = -1;
    if (live && lane < k) {
        int c = -1;
        if ((unsigned)my_e < (unsigned)E) {
            const int cand = s_base[my_e] + my_rank;
            if (cand < C) {
                c = cand;
                myrow = s_off[my_e] + cand;
                src_token[myrow] = (int32_t)t;
            }
        }
        slot[t * k + lane] = c;
        row_of[t * k + lane] = myrow;
    }
    if (live) {
        for (int r = 0; r < k; ++r) {
            const int row = lane_value(myrow, r);   // uniform over the wave
            if (row < 0) continue;
            V* dst = x_perm + (int64_t)row * vec_per_row;
#pragma unroll
            for (int u = 0; u < NPF; ++u) {
                const int64_t c = (int64_t)u * 64 + lane;
                if (c < vec_per_row) dst[c] = v[u];
            }
        }
        // uniform trip count: every lane stays active around lane_value
        for (int64_t c0 = (int64_t)NPF * 64; c0 < vec_per_row; c0 += 64) {
            const int64_t c = c0 + lane;
            const bool ok = c < vec_per_row;
            V w;
            if (ok) w = src[c];
            for (int r = 0; r < k; ++r) {
                const int row = lane_value(myrow, r);
                if (row >= 0 && ok) x_perm[(int64_t)row * vec_per_row + c] = w;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Overflow variant: rerouting a rejected path to the next-choice expert
// ("The real cost of sparse expert models" item 5; ch. 36 §36.3 overflow
// treatments).  Read as: the candidates are accepted first, in token order
// (Algorithm 36.1); then the j-th rejected candidate of each token, in rank
// order, asks for the token's j-th next expert, in token order, into the
// capacity left; rejected again, it is dropped.  Every second-pass request comes
// after every first-pass one, so running the ordinary dispatch over 2T "tokens"
// -- the candidates, then each token's spare requests -- gives exactly these
// slots: an expert with L_e < C accepts the spare requests while L_e + (earlier
// spare requests) < C, one with L_e >= C none, as the definition says.
// ---------------------------------------------------------------------------

// v[t][r] = ids[t][r] (r < k): the candidates of the P = 2k routing records.
__global__ __launch_bounds__(256) void reroute_candidates_kernel(const int32_t* __restrict__ ids, int64_t T, int k,
                                                                 int32_t* __restrict__ v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * k) return;
    v[i] = ids[(i / k) * 2 * k + i % k];
}

// v[T + t][j] = ids[t][k + j] for the first (number of rejected candidates) j,
// else -1 (no request); slot1: the first pass's slots [T][k].
__global__ __launch_bounds__(256) void reroute_requests_kernel(const int32_t* __restrict__ ids, int64_t T, int k,
                                                               const int32_t* __restrict__ slot1,
                                                               int32_t* __restrict__ v) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    int nrej = 0;
    for (int r = 0; r < k; ++r) nrej += slot1[t * k + r] < 0;
    for (int j = 0; j < k; ++j) v[(T + t) * k + j] = j < nrej ? ids[t * 2 * k + k + j] : -1;
}

// One workgroup: the 2T-token run's slots and rows folded back to [T][2k]
// (candidate r at column r, spare j at column k + j), the spare rows' source
// token, and the statistics (O and max load from the first pass, accepted rows
// from the second, rerouted paths, tokens affected / left with no path).
__global__ __launch_bounds__(1024) void reroute_finish_kernel(int64_t T, int k, const int32_t* __restrict__ slot2,
                                                              const int32_t* __restrict__ row2,
                                                              const int32_t* __restrict__ stats1,
                                                              const int32_t* __restrict__ stats2,
                                                              int32_t* __restrict__ slot, int32_t* __restrict__ row_of,
                                                              int32_t* __restrict__ src_token,
                                                              int32_t* __restrict__ stats) {
    __shared__ int s_sum[3][16];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    int rerouted = 0, affected = 0, dropped = 0;
    for (int64_t t = tid; t < T; t += 1024) {
        int served = 0, nrej = 0;
        for (int r = 0; r < k; ++r) {
            const int c = slot2[t * k + r], rw = row2[t * k + r];
            slot[t * 2 * k + r] = c;
            row_of[t * 2 * k + r] = rw;
            served += c >= 0;
            nrej += c < 0;
        }
        for (int j = 0; j < k; ++j) {
            const int c = slot2[(T + t) * k + j], rw = row2[(T + t) * k + j];
            slot[t * 2 * k + k + j] = c;
            row_of[t * 2 * k + k + j] = rw;
            if (rw >= 0) {
                src_token[rw] = (int32_t)t;
                ++rerouted;
                ++served;
            }
        }
        affected += nrej > 0;
        dropped += served == 0;
    }
    int v[3] = {rerouted, affected, dropped};
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        for (int o = 32; o >= 1; o >>= 1) v[q] += __shfl_xor(v[q], o, MOE_WAVE);
        if (lane == 0) s_sum[q][wave] = v[q];
    }
    __syncthreads();
    if (tid == 0) {
        int tot[3] = {0, 0, 0};
        for (int q = 0; q < 3; ++q)
            for (int w = 0; w < 16; ++w) tot[q] += s_sum[q][w];
        for (int i = 0; i < MOE_STAT_COUNT; ++i) stats[i] = 0;
        stats[MOE_STAT_OVERFLOW] = stats1[MOE_STAT_OVERFLOW];
        stats[MOE_STAT_ACCEPTED] = stats2[MOE_STAT_ACCEPTED];
        stats[MOE_STAT_MAX_LOAD] = stats1[MOE_STAT_MAX_LOAD];
        stats[MOE_STAT_REROUTED] = tot[0];
        stats[MOE_STAT_TOKENS_AFFECTED] = tot[1];
        stats[MOE_STAT_TOKENS_DROPPED] = tot[2];
    }
}

// Load-balance statistics ("LLM from scratch" ch. 36 §36.4 and its worked
// example): f_e = L_e / (T k), the pre-capacity share of routing records;
// p_bar_e = prob_sum_e / T, the mean full-softmax probability; the balance value
// E sum_e f_e p_bar_e (1 at the uniform point); the path rejection rate O / (T k),
// the shares of tokens with some / all paths rejected, and rho_max = max_e L_e /
// (T k / E) ("The real cost of sparse expert models", load ratio).  One
// workgroup, E <= 1024; the sum over e runs in a fixed order.
__global__ __launch_bounds__(1024) void balance_kernel(const int32_t* __restrict__ load,
                                                       const int32_t* __restrict__ stats,
                                                       const float* __restrict__ prob_sum, int64_t T, int E, int k,
                                                       float* __restrict__ out) {
    __shared__ float part[16];
    const int e = threadIdx.x, wave = e / 64, lane = e % 64;
    const double paths = (double)T * k;
    float f = 0.f, p = 0.f;
    if (e < E && T > 0) {
        f = (float)(load[e] / paths);
        p = (float)(prob_sum[e] / (double)T);
    }
    if (e < E) {
        out[e] = f;
        out[E + e] = p;
    }
    float fp = f * p;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) fp += __shfl_xor(fp, o, MOE_WAVE);
    if (lane == 0) part[wave] = fp;
    __syncthreads();
    if (e == 0) {
        float sum = 0.f;
        for (int w = 0; w < 16; ++w) sum += part[w];
        const bool any = T > 0;
        out[2 * E + MOE_BAL_VALUE] = (float)E * sum;
        out[2 * E + MOE_BAL_PATH_REJECTION] = any ? (float)(stats[MOE_STAT_OVERFLOW] / paths) : 0.f;
        out[2 * E + MOE_BAL_TOKENS_AFFECTED] = any ? (float)(stats[MOE_STAT_TOKENS_AFFECTED] / (double)T) : 0.f;
        out[2 * E + MOE_BAL_TOKENS_DROPPED] = any ? (float)(stats[MOE_STAT_TOKENS_DROPPED] / (double)T) : 0.f;
        out[2 * E + MOE_BAL_RHO_MAX] = any ? (float)(stats[MOE_STAT_MAX_LOAD] / (paths / E)) : 0.f;
    }
}

}  // namespace

namespace moe_kernels {

hipError_t launch_balance(const moe_dims& s, const int32_t* load, const int32_t* stats, const float* prob_sum,
                          float* out, hipStream_t st) {
    hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(1024), 0, st, load, stats, prob_sum, s.T, s.E, s.k, out);
    return hipGetLastError();
}


namespace {
inline size_t al8(size_t v) { return (v + 7) / 8 * 8; }
}

bool dispatch_uses_hist(const moe_dims& s) { return s.accept_by_gate || s.T > DB_TOK; }

bool dispatch_inline_scan(const moe_dims& s) {
    const int64_t NB = (s.T + DB_TOK - 1) / DB_TOK;
    return !s.accept_by_gate && NB > 1 && s.E <= DB_TOK && NB * s.E <= SCAN_INLINE_MAX;
}

bool dispatch_router_counts_ok(const moe_dims& s) {
    return !s.reroute && dispatch_inline_scan(s) && (s.T + MOE_ROUTE_TOK - 1) / MOE_ROUTE_TOK * s.E <= SCAN_INLINE_MAX;
}

namespace {
// The rerouting dispatch's two ordinary runs: over the T candidates' tokens, and
// over 2T tokens (candidates, then spare requests).
moe_dims reroute_pass(const moe_dims& s, int64_t T) {
    moe_dims r = s;
    r.T = T;
    r.reroute = 0;
    return r;
}
// [v 2Tk | slot1, row1 Tk | src1 | offsets1 E+1 | stats1, stats2 | load2 E | slot2, row2 2Tk | run workspace]
struct RerouteWs {
    int32_t *v, *slot1, *row1, *src1, *off1, *stats1, *stats2, *load2, *slot2, *row2;
    void* run;
    size_t total;
};
RerouteWs carve_reroute(const moe_dims& s, void* base) {
    RerouteWs w{};
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t n) -> int32_t* {
        int32_t* r = p ? reinterpret_cast<int32_t*>(p + off) : nullptr;
        off += al8(n * sizeof(int32_t));
        return r;
    };
    const int64_t Tk = s.T * s.k;
    const moe_dims s1 = reroute_pass(s, s.T), s2 = reroute_pass(s, 2 * s.T);
    w.v = take(2 * Tk);
    w.slot1 = take(Tk);
    w.row1 = take(Tk);
    w.src1 = take(Tk < (int64_t)s.E * s.C ? Tk : (int64_t)s.E * s.C);
    w.off1 = take(s.E + 1);
    w.stats1 = take(MOE_STAT_COUNT);
    w.stats2 = take(MOE_STAT_COUNT);
    w.load2 = take(s.E);
    w.slot2 = take(2 * Tk);
    w.row2 = take(2 * Tk);
    off = (off + 255) & ~(size_t)255;
    w.run = p ? p + off : nullptr;
    const size_t a = dispatch_ws_bytes(s1), b = dispatch_ws_bytes(s2);
    w.total = off + (a > b ? a : b);
    return w;
}
}  // namespace

size_t dispatch_ws_bytes(const moe_dims& s) {
    if (s.reroute) return carve_reroute(s, nullptr).total;
    const int64_t NB = (s.T + DB_TOK - 1) / DB_TOK;
    const int64_t rows = dispatch_router_counts_ok(s) ? (s.T + MOE_ROUTE_TOK - 1) / MOE_ROUTE_TOK : NB;
    size_t b = al8((size_t)rows * (size_t)s.E * sizeof(int32_t));   // per-block (or router-group) counts / bases
    if (s.accept_by_gate) {
        // request offsets, thresholds, request keys and path ids
        b += al8(sizeof(int32_t) * (s.E + 1)) + sizeof(unsigned long long) * s.E +
             (sizeof(unsigned long long) + sizeof(int32_t)) * (size_t)s.T * s.k;
    }
    return b;
}

hipError_t launch_dispatch(const moe_dims& s, const void* x, const int32_t* ids, const float* topk_w, int32_t* load,
                           int32_t* offsets, int32_t* slot, int32_t* row_of, int32_t* src_token, void* x_perm,
                           int32_t* stats, void* ws, hipStream_t st, int32_t* tprefix, int tile_rows,
                           bool hist_ready, int32_t* status, int32_t* route_flag) {
    const int NB = (int)((s.T + DB_TOK - 1) / DB_TOK);
    int32_t* hist = static_cast<int32_t*>(ws);
    const size_t mask_lds = sizeof(unsigned long long) * 4 * s.E;
    if (s.reroute) {
        if (s.T == 0) return launch_dispatch(reroute_pass(s, 0), x, ids, topk_w, load, offsets, slot, row_of,
                                             src_token, nullptr, stats, ws, st, tprefix, tile_rows);
        const RerouteWs w = carve_reroute(s, ws);
        const int64_t Tk = s.T * s.k;
        hipLaunchKernelGGL(reroute_candidates_kernel, dim3((unsigned)((Tk + 255) / 256)), dim3(256), 0, st, ids, s.T,
                           s.k, w.v);
        // first pass: the candidates alone give L_e (the requested load), O, the max load and the rejections
        hipError_t e = launch_dispatch(reroute_pass(s, s.T), x, w.v, nullptr, load, w.off1, w.slot1, w.row1, w.src1,
                                       nullptr, w.stats1, w.run, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(reroute_requests_kernel, dim3((unsigned)((s.T + 255) / 256)), dim3(256), 0, st, ids, s.T,
                           s.k, w.slot1, w.v);
        // second pass over 2T tokens: the final slots, rows, offsets and the GEMMs' tile prefix
        e = launch_dispatch(reroute_pass(s, 2 * s.T), x, w.v, nullptr, w.load2, offsets, w.slot2, w.row2, src_token,
                            nullptr, w.stats2, w.run, st, tprefix, tile_rows);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(reroute_finish_kernel, dim3(1), dim3(1024), 0, st, s.T, s.k, w.slot2, w.row2, w.stats1,
                           w.stats2, slot, row_of, src_token, stats);
    } else if (s.accept_by_gate) {
        char* p = static_cast<char*>(ws) + al8((size_t)NB * s.E * sizeof(int32_t));
        int32_t* roff = reinterpret_cast<int32_t*>(p);
        p += al8(sizeof(int32_t) * (s.E + 1));
        unsigned long long* thresh = reinterpret_cast<unsigned long long*>(p);
        p += sizeof(unsigned long long) * s.E;
        unsigned long long* req_key = reinterpret_cast<unsigned long long*>(p);
        p += sizeof(unsigned long long) * (size_t)s.T * s.k;
        int32_t* req_path = reinterpret_cast<int32_t*>(p);
        if (NB > 0)
            hipLaunchKernelGGL(dispatch_count_kernel, dim3(NB), dim3(DB_TOK), mask_lds, st, ids, s.T, s.k, s.E,
                               hist, (int32_t*)nullptr, (int32_t*)nullptr);
        hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, hist, NB, s.E, s.C, load, offsets,
                           stats, tprefix, tile_rows, roff);
        if (NB == 0) return hipGetLastError();
        hipLaunchKernelGGL(dispatch_requests_kernel, dim3(NB), dim3(DB_TOK), mask_lds, st, ids, topk_w, s.T, s.k,
                           s.E, hist, roff, req_key, req_path, slot, row_of);
        hipLaunchKernelGGL(dispatch_threshold_kernel, dim3(s.E), dim3(1024), 0, st, load, roff, s.C, req_key,
                           thresh);
        hipLaunchKernelGGL(dispatch_assign_kernel, dim3(s.E), dim3(1024), 0, st, load, roff, offsets, s.k, req_key,
                           req_path, thresh, slot, row_of, src_token);
        hipLaunchKernelGGL(dispatch_token_stats_kernel, dim3(NB), dim3(DB_TOK), 0, st, row_of, s.T, s.k, stats);
    } else if (NB == 1) {
        hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), mask_lds + sizeof(int) * s.E, st, ids, s.T,
                           s.k, s.E, s.C, load, offsets, stats, tprefix, tile_rows, slot, row_of, src_token);
    } else if (NB > 0 && dispatch_inline_scan(s) && !hist_ready && x_perm) {
        // standalone, with the row copy: count (table and ranks), then placement + gather
        hipLaunchKernelGGL(dispatch_count_kernel, dim3(NB), dim3(DB_TOK), mask_lds, st, ids, s.T, s.k, s.E, hist,
                           stats + MOE_STAT_TOKENS_DROPPED, slot);
        const int elem = s.dtype == MOE_BF16 ? 2 : 4;
        const int64_t row_bytes = (int64_t)s.d * elem;
        const unsigned grid = (unsigned)((s.T + 3) / 4);
        const size_t lds = sizeof(int32_t) * (2 + (size_t)NB) * s.E;
        if (row_bytes % 16 == 0)
            hipLaunchKernelGGL((dispatch_place_gather_kernel<u32x4, 8>), dim3(grid), dim3(256), lds, st,
                               static_cast<const u32x4*>(x), ids, s.T, s.k, s.E, s.C, hist, NB, load, offsets, slot,
                               row_of, src_token, stats, tprefix, tile_rows, row_bytes / 16,
                               static_cast<u32x4*>(x_perm));
        else   // fp32 rows (bf16 rows are whole 16-byte chunks: d % 8 == 0)
            hipLaunchKernelGGL((dispatch_place_gather_kernel<uint32_t, 8>), dim3(grid), dim3(256), lds, st,
                               static_cast<const uint32_t*>(x), ids, s.T, s.k, s.E, s.C, hist, NB, load, offsets,
                               slot, row_of, src_token, stats, tprefix, tile_rows, row_bytes / 4,
                               static_cast<uint32_t*>(x_perm));
        // with distinct ids per token no path is rejected unless C < T (the
        // counters stay as the count kernel cleared them)
        if (s.C < s.T)
            hipLaunchKernelGGL(dispatch_token_stats_kernel, dim3(NB), dim3(DB_TOK), 0, st, row_of, s.T, s.k, stats);
        return hipGetLastError();
    } else if (NB > 0 && dispatch_inline_scan(s)) {
        // the token statistics are accumulated by the placement into counters the
        // table's writer clears (here the count kernel, else the router, whose
        // table has one row per MOE_ROUTE_TOK tokens)
        if (!hist_ready)
            hipLaunchKernelGGL(dispatch_count_kernel, dim3(NB), dim3(DB_TOK), mask_lds, st, ids, s.T, s.k, s.E,
                               hist, stats + MOE_STAT_TOKENS_DROPPED, (int32_t*)nullptr);
        const int sub = hist_ready ? DB_TOK / MOE_ROUTE_TOK : 1;
        const int NR = hist_ready ? (int)((s.T + MOE_ROUTE_TOK - 1) / MOE_ROUTE_TOK) : NB;
        const size_t lds = mask_lds + sizeof(int32_t) * (2 * s.E + (size_t)NR * s.E);
        hipLaunchKernelGGL(dispatch_place_scan_kernel, dim3(NB), dim3(DB_TOK), lds, st, ids, s.T, s.k, s.E, s.C,
                           hist, NR, sub, load, offsets, slot, row_of, src_token, stats, tprefix, tile_rows,
                           hist_ready ? status : nullptr, route_flag);
    } else {
        if (NB > 0) {
            hipLaunchKernelGGL(dispatch_count_kernel, dim3(NB), dim3(DB_TOK), mask_lds, st, ids, s.T, s.k, s.E,
                               hist, (int32_t*)nullptr, (int32_t*)nullptr);
        }
        hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, hist, NB, s.E, s.C, load, offsets,
                           stats, tprefix, tile_rows, (int32_t*)nullptr);
        if (NB == 0) return hipGetLastError();
        hipLaunchKernelGGL(dispatch_place_kernel, dim3(NB), dim3(DB_TOK), mask_lds, st, ids, s.T, s.k, s.E, s.C,
                           hist, offsets, slot, row_of, src_token, stats);
    }
    if (!x_perm) return hipGetLastError();
    const int elem = s.dtype == MOE_BF16 ? 2 : 4;
    const int64_t row_bytes = (int64_t)s.d * elem;
    const unsigned grid = (unsigned)((s.T + 3) / 4);
    const int P = moe_paths(s);   // routing records per token
    if (row_bytes % 16 == 0)
        hipLaunchKernelGGL(dispatch_gather_kernel<uint4>, dim3(grid), dim3(256), 0, st, static_cast<const uint4*>(x),
                           s.T, P, row_bytes / 16, row_of, static_cast<uint4*>(x_perm));
    else   // fp32 rows (bf16 rows are whole 16-byte chunks: d % 8 == 0)
        hipLaunchKernelGGL(dispatch_gather_kernel<uint32_t>, dim3(grid), dim3(256), 0, st,
                           static_cast<const uint32_t*>(x), s.T, P, row_bytes / 4, row_of,
                           static_cast<uint32_t*>(x_perm));
    return hipGetLastError();
}

}  // namespace moe_kernels
