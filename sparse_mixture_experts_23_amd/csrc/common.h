// Shared device helpers for the gfx950 (CDNA4) MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

#include "../../include/moe.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand (8 x K)
typedef __attribute__((ext_vector_type(4))) float floatx4_t;    // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(16))) float floatx16_t;  // 32x32 MFMA accumulator

#define MOE_WAVE 64

// bf16 is carried as its 16-bit pattern in memory.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// fp32 -> bf16 bit pattern, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z); e^-z from the hardware exp2.
__device__ __forceinline__ float silu_f32(float z) {
    // hardware exp2 and reciprocal (<= 1 ulp each) instead of an IEEE division
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Two floats to packed bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float floatx2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const floatx2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Total order on finite floats as unsigned keys (larger float -> larger key);
// -0.0 is mapped to +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t float_order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Value of `v` in lane `lane` (wave-uniform), read with v_readlane: unlike a
// shuffle it does not depend on which lanes are active at the call site, so it
// is safe inside lane-divergent loops as long as `v` was written before them.
__device__ __forceinline__ int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float lane_value(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        unsigned long long w = __shfl_xor(v, o, MOE_WAVE);
        v = w > v ? w : v;
    }
    return v;
}

// ---- host-side launch helpers shared by the translation units ----------------

struct moe_dims {
    int64_t T;
    int d, m, E, k;
    int C;          // effective capacity (T when unlimited)
    int gate_mode;
    int dtype;
    int m_shared;
    int accept_by_gate;     // overflow variant: acceptance by routing weight
    int renorm_survivors;   // overflow variant: weights renormalised over accepted paths
    int reroute;            // overflow variant: rejected paths go to the next-choice expert
};

// Routing records per token: the k selected experts, and with rerouting the next
// k in rank order as well.
inline int moe_paths(const moe_dims& s) { return s.reroute ? 2 * s.k : s.k; }

// Tokens per block of the dispatch's per-block expert counts, hist[b][e] = number
// of tokens in [256 b, 256 b + 256) that selected expert e.
constexpr int MOE_DISPATCH_BLOCK = 256;

// Tokens per workgroup of the E <= 8 router, and so per row of the expert counts
// it makes for the dispatch.  Its sync words, MOE_SYNC_BYTES at the start of every
// route, route-stats and forward workspace: [0] workgroups finished, [1]
// non-finite flag.
constexpr int MOE_ROUTE_TOK = 16;

// Work-claim counters of the grouped bf16 GEMMs, kept after the tile prefix
// (tprefix[0..G]) in the same workspace: MOE_SCHED_WORDS 64-bit words, one per
// XCD for GEMM1, then one per XCD for GEMM2.  Every kernel that writes a tile
// prefix also clears them, so each GEMM launch starts from zero.
constexpr int MOE_SCHED_WORDS = 16;
__host__ __device__ inline unsigned long long* moe_sched_words(int32_t* tprefix, int G) {
    return reinterpret_cast<unsigned long long*>(tprefix + ((G + 2) & ~1));
}

namespace moe_kernels {

// Router: scores, softmax, top-k, weights.  ws holds the weight planes or the
// fp32 scores (route_ws_bytes).  sync: the MOE_SYNC_BYTES of sync words (zero on
// entry, zero again when the launch ends), used by the E <= 8 path.
// probs (nullable): also write every token's full softmax, probs[t E + e].
// hist (nullable): the dispatch's expert counts per MOE_ROUTE_TOK tokens
// ([ceil(T / MOE_ROUTE_TOK)][E] int32, dispatch_router_counts_ok).  Where the
// router path counts them while it selects (E <= 8), it fills them, clears the
// two counters at acc_stats and sets *hist_done; otherwise it leaves them alone.
// With *hist_done set, the status word is not written here: the router only
// raises the flag in sync[1], and launch_dispatch (given status and that flag)
// writes the status and clears the flag.
size_t route_ws_bytes(const moe_dims& s);
hipError_t launch_route(const moe_dims& s, const void* x, const float* w_r, const float* b_r,
                        int32_t* topk_ids, float* topk_w, int32_t* status, void* ws, int32_t* sync, hipStream_t st,
                        float* probs = nullptr, int32_t* hist = nullptr, bool* hist_done = nullptr,
                        int32_t* acc_stats = nullptr);
// Small batches (bf16, 0 < T <= 16, E <= 256, acceptance in token order): route,
// dispatch and row gather of the whole layer front in one workgroup (after a
// split-K dot kernel for E > 8); the same outputs as launch_route followed by
// launch_dispatch, and the GEMMs' tile prefix in tprefix.  ws: route_ws_bytes.
// x_perm == nullptr: no row copy.
bool front_fused_ok(const moe_dims& s);
hipError_t launch_front(const moe_dims& s, const void* x, const float* w_r, const float* b_r, int32_t* topk_ids,
                        float* topk_w, int32_t* status, void* ws, hipStream_t st, int32_t* load, int32_t* offsets,
                        int32_t* slot, int32_t* row_of, int32_t* src_token, void* x_perm, int32_t* stats,
                        int32_t* tprefix, int tile_rows);
// prob_sum[e] = sum_t probs[t E + e] in a fixed order.
hipError_t launch_prob_sum(const moe_dims& s, const float* probs, float* prob_sum, hipStream_t st);
// Balance statistics from the loads, the dispatch statistics and prob_sum (out: see moe_balance).
hipError_t launch_balance(const moe_dims& s, const int32_t* load, const int32_t* stats, const float* prob_sum,
                          float* out, hipStream_t st);

// dst[b][j][i] = src[b][i][j] over batch matrices of rows x cols elements of
// elem_bytes (2 or 4); grid limits: batch <= 65535, rows <= 65535 x 64.
hipError_t launch_transpose(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols, int elem_bytes,
                            hipStream_t st);

// Dispatch.
size_t dispatch_ws_bytes(const moe_dims& s);
// Whether launch_dispatch reads the per-block expert counts (more than one token
// block, or acceptance by gate weight); a single block is counted in place.
bool dispatch_uses_hist(const moe_dims& s);
// Whether launch_dispatch can take the counts per MOE_ROUTE_TOK tokens from the
// router (the inline scan, with a table of at most SCAN_INLINE_MAX entries).
bool dispatch_router_counts_ok(const moe_dims& s);
// Whether launch_dispatch derives the scan inside the placement kernel (a small
// count table); the placement then accumulates the token statistics into
// stats[MOE_STAT_TOKENS_DROPPED..AFFECTED], which whoever fills the table clears.
bool dispatch_inline_scan(const moe_dims& s);
// tprefix (nullable): also write the grouped GEMMs' tile prefix for tiles of
// tile_rows rows (gemm_tile_rows), so the GEMM launches can skip computing it.
// topk_w: the routing weights (read only when s.accept_by_gate).
// ws starts with the per-block expert counts (dispatch_hist); hist_ready: the
// router has already written them per MOE_ROUTE_TOK tokens
// (dispatch_router_counts_ok), so the counting kernel is skipped.  x_perm
// == nullptr: no row copy (the caller reads x through src_token).  status /
// route_flag (with hist_ready): the router left its non-finite flag at route_flag
// instead of writing the status; the placement writes *status from it and clears it.
hipError_t launch_dispatch(const moe_dims& s, const void* x, const int32_t* ids, const float* topk_w,
                           int32_t* load, int32_t* offsets, int32_t* slot, int32_t* row_of, int32_t* src_token,
                           void* x_perm, int32_t* stats, void* ws, hipStream_t st,
                           int32_t* tprefix = nullptr, int tile_rows = 0, bool hist_ready = false,
                           int32_t* status = nullptr, int32_t* route_flag = nullptr);

// Grouped expert GEMMs.  offsets == nullptr means one group covering rows [0, nrows).
size_t gemm_ws_bytes(int G);
// ws starts with the tile prefix of `offsets` (G + 1 int32, gemm_ws_bytes); it is
// computed by the launch unless prefix_ready (then the caller wrote it, e.g. the
// dispatch scan).
int gemm_tile_rows(int dtype);
// GEMM1 may split K over S = gemm1_splits(...) workgroups per tile when few row
// tiles exist (decided from the shape alone); it then needs `part`, fp32 scratch
// of gemm1_part_bytes(...) (S gate and S up partials), and forms h from their
// sums.  With part == nullptr it never splits.
// group_rows: an upper bound on the rows of any one group (the routed experts:
// min(T, C), a token adding at most one row per expert; the shared expert: T).
// With at most MOE_GEMV_ROWS rows per group (decode batches) both GEMMs run as
// grouped GEMVs that stream the active groups' weights, and never split K.
constexpr int64_t MOE_GEMV_ROWS = 8;
constexpr int64_t MOE_ROWS_UNKNOWN = INT64_MAX;
bool gemv_path(int dtype, int64_t group_rows);
int gemm1_splits(int dtype, int64_t max_rows, int G, int N, int K, int64_t group_rows = MOE_ROWS_UNKNOWN);
size_t gemm1_part_bytes(int dtype, int64_t max_rows, int G, int N, int K, int64_t group_rows = MOE_ROWS_UNKNOWN);
// gather (nullable, only where gemm1_gather_ok): A is the token-ordered [a_rows, K]
// activations and grouped row r reads A row gather[r] (the dispatch's src_token,
// readable up to 256 entries past the last row), so no grouped copy is needed.
bool gemm1_gather_ok(int dtype, int N, int K, int64_t a_rows);
hipError_t launch_gemm1(int dtype, const void* A, const int32_t* offsets, int G, int64_t max_rows,
                        const void* w_gate, const void* w_up, void* h, int N, int K,
                        void* ws, hipStream_t st, bool prefix_ready = false, float* part = nullptr,
                        const int32_t* gather = nullptr, int64_t group_rows = MOE_ROWS_UNKNOWN);
// GEMM2 may split K over S = gemm2_splits(...) (decided from the shape alone):
// then H receives the partial sum over the first K range and H1 + (s - 1) max_rows N
// the sum over range s = 1..S-1; with H1 == nullptr it never splits.
int gemm2_splits(int dtype, int64_t max_rows, int G, int N, int K, int64_t group_rows = MOE_ROWS_UNKNOWN);
hipError_t launch_gemm2(int dtype, const void* h, const int32_t* offsets, int G, int64_t max_rows,
                        const void* w_down, float* H, float* H1, int N, int K, void* ws, hipStream_t st,
                        bool prefix_ready = false, int64_t group_rows = MOE_ROWS_UNKNOWN);
// H += H1[0] + ... + H1[np - 1] (blocks of max_rows N floats, added in order) over the
// rows [0, offsets[G]) (or [0, max_rows) without offsets); N % 4 == 0.
hipError_t launch_add_partial(float* H, const float* H1, int np, const int32_t* offsets, int G, int64_t max_rows,
                              int N, hipStream_t st);

// Ungrouped bf16 GEMM part[s] = x[T,K] . w[N,K]^T over the K split s of
// scores_splits(T, N, K) splits; part holds S consecutive fp32 [T,N] blocks.
int scores_splits(int64_t T, int N, int K);
hipError_t launch_scores_gemm(const void* x, const void* w, int64_t T, int N, int K, float* part, hipStream_t st);

// Combine.  H1 (nullable): np further K-split partials of H (blocks of
// part_stride floats), added to the H row in order before weighting.
hipError_t launch_combine(const moe_dims& s, const float* H, const float* H1, int np, int64_t part_stride,
                          const int32_t* row_of, const float* topk_w, const float* shared_out, float* y,
                          hipStream_t st);

}  // namespace moe_kernels
