/*
 * moe.h -- C-ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward.
 *
 * The layer (one routing group of T valid tokens):
 *   router scores  g = x W_r^T + b_r, softmax over the experts
 *       ("LLM from scratch" ch. 36 §36.1; "MoE token routing" §2)
 *   top-k          k distinct experts by descending score, ties to the lower id
 *       (ch. 36 §36.1 and Algorithm 36.1 in §36.4)
 *   weights        renormalised within the selected set, or the Switch
 *                  convention that keeps the full-softmax probability
 *       (ch. 36 §36.2)
 *   dispatch       capacity C per expert, slots first-come-first-served in
 *                  token order, overflowing paths rejected (contribute 0,
 *                  no second renormalisation)
 *       (ch. 36 §36.3 and Algorithm 36.1; "The real cost of sparse expert
 *        models" equation for C_e and O); two overflow variants are shape
 *       fields: acceptance by gate weight, weights renormalised over the
 *       surviving paths (ch. 36 §36.3-§36.4)
 *   experts        SwiGLU  E_i(x) = [SiLU(x W_gate,i) (*) (x W_up,i)] W_down,i
 *       ("MoE token routing" §3)
 *   shared expert  optional, applied to every token, unweighted
 *       (ch. 36 §36.6; "Sizzling MoE skewer analogy" DeepSeek-V3 formula)
 *   combine        y_t = s_t + sum over accepted paths of a_te * H_e[slot]
 *       (Algorithm 36.1; "MoE token routing" §3)
 *   statistics     requested load L_e, accepted, overflow O, max load,
 *                  tokens affected / fully dropped; rho_max = max L_e/(Tk/E)
 *       (ch. 36 §36.4; "The real cost of sparse expert models" equations)
 *
 * Conventions common to every call:
 *  - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *    owns every buffer; the library never allocates or frees memory and keeps
 *    no per-call state.  Inputs and outputs must not alias.
 *  - Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *    void*, NULL = the null stream).  Argument errors are detected on the host,
 *    before anything is launched, and returned synchronously.
 *  - Expert ids are 0-based.  Matrices are row-major.  Weights are stored
 *    out-features x in-features (the transpose convention ch. 36 §36.8
 *    mentions): router w_r [E,d], gate/up [E,m,d], down [E,d,m].
 *  - dtype MOE_F32: x, expert weights, h are fp32.  MOE_BF16: x and expert
 *    weights are bf16, h is bf16; all accumulation is fp32.  The router
 *    weights, bias, routing weights, H, s and y are always fp32.
 *  - y excludes the residual: a token whose every path is rejected gets
 *    y_t = s_t (0 without a shared expert); the caller adds its residual.
 *  - Calls are reentrant; concurrent calls must use disjoint buffers.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,   /* bad shape, pointer, k or capacity      */
    MOE_ERR_NONFINITE_LOGIT = 2,    /* written to the device status word only */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_UNSUPPORTED = 4,        /* valid but outside the supported shapes */
    MOE_ERR_HIP = 5                 /* a HIP runtime call or launch failed    */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_GATE_RENORM = 0, MOE_GATE_SWITCH = 1 } moe_gate_mode;

/* Layer shape.  capacity: C >= 1, or 0 = unlimited (no path can be rejected).
 * Supported: T >= 0; d, m >= 1; 1 <= k <= E <= 1024, k <= 32; for MOE_BF16 d
 * and m must be multiples of 8 (16-byte rows).  m_shared: 0 = no shared
 * expert, else its width (same alignment rule). */
typedef struct {
    int64_t T;
    int32_t d, m, E, k;
    int32_t capacity;
    int32_t gate_mode;   /* moe_gate_mode */
    int32_t dtype;       /* moe_dtype     */
    int32_t m_shared;
    /* Overflow variants (ch. 36 §36.3 acceptance rules and overflow; §36.4 worked
     * example); both 0 is the chapter's Algorithm 36.1:
     *   accept_by_gate   1: an expert over capacity keeps the C requests with the
     *                    largest routing weight (equal weights: earlier token),
     *                    instead of the first C in token order; accepted rows
     *                    still keep token order inside the expert's group
     *   renorm_survivors 1: the combine divides each accepted weight by the sum
     *                    of the token's accepted weights (a token with no
     *                    accepted path still adds nothing) */
    int32_t accept_by_gate;
    int32_t renorm_survivors;
    /* reroute 1: a path its expert rejects asks for the token's next-choice
     * expert instead ("The real cost of sparse expert models" item 5; ch. 36
     * §36.3 overflow treatments; read here as: the j-th rejected candidate of a
     * token, in rank order, asks for its j-th next expert in rank order; these
     * requests are accepted in token order, after every first-pass request, into
     * the capacity left; a path rejected again is dropped).  The routing records
     * (topk_ids, topk_w, slot, row_of) then have P = 2k columns per token: the
     * k selected experts, then the next k in rank order (id -1, weight 0 where
     * the experts run out).  A next-choice path's weight is its expert's gate
     * value with the selection's normalizer (RENORM p_e' / sum_{j in S_t} p_j,
     * SWITCH p_e').  Requires accept_by_gate == 0. */
    int32_t reroute;
} moe_shape;

/* Indices of the int32 statistics vector written by moe_dispatch. */
enum {
    MOE_STAT_OVERFLOW = 0,        /* O = sum_e max(0, L_e - C) = rejected paths   */
    MOE_STAT_ACCEPTED = 1,        /* A = sum_e min(L_e, C): rows of x_perm / H    */
    MOE_STAT_MAX_LOAD = 2,        /* max_e L_e (requested, before capacity)      */
    MOE_STAT_TOKENS_DROPPED = 3,  /* tokens with every path rejected             */
    MOE_STAT_TOKENS_AFFECTED = 4, /* tokens with at least one path rejected      */
    MOE_STAT_REROUTED = 5,        /* with reroute: rejected paths served by a
                                     next-choice expert (O counts the first pass) */
    MOE_STAT_COUNT = 8
};

/* Indices, after the 2E per-expert values, of the fp32 vector written by
 * moe_balance. */
enum {
    MOE_BAL_VALUE = 0,            /* E * sum_e f_e * p_bar_e (1 at the uniform point) */
    MOE_BAL_PATH_REJECTION = 1,   /* O / (T k)                                        */
    MOE_BAL_TOKENS_AFFECTED = 2,  /* tokens with at least one path rejected / T       */
    MOE_BAL_TOKENS_DROPPED = 3,   /* tokens with every path rejected / T              */
    MOE_BAL_RHO_MAX = 4,          /* max_e L_e / (T k / E)                            */
    MOE_BAL_COUNT = 5
};

/* Bytes at the start of every route, route-stats and forward workspace that
 * hold the router's completion counters.  They must be zero before the first
 * call that uses the workspace (clear them once when the buffer is allocated)
 * and must not be used for anything else; every call leaves them at zero. */
#define MOE_SYNC_BYTES 256

/* Which call a workspace is sized for. */
typedef enum {
    MOE_WS_DISPATCH = 0, MOE_WS_FFN = 1, MOE_WS_SHARED = 2, MOE_WS_FORWARD = 3, MOE_WS_ROUTE = 4,
    MOE_WS_ROUTE_STATS = 5
} moe_ws_kind;

/* ---- host helpers ------------------------------------------------------ */

/* Capacity C = ceil(cf * T * k / E) with cf = cf_num / cf_den, in exact
 * integer arithmetic ("The real cost of sparse expert models", equation for
 * C_e; ch. 36 §36.3; "MoE token routing" §6).  Returns -1 on invalid input
 * (T < 0, k < 1, E < 1, cf_num < 1, cf_den < 1) or if C exceeds INT32_MAX. */
int32_t moe_capacity(int64_t T, int32_t k, int32_t E, int32_t cf_num, int32_t cf_den);

/* Upper bound on the accepted paths A = rows of x_perm / h / H:
 * min(T*k, E*C) (C = T when unlimited).  0 for an invalid shape. */
int64_t moe_max_rows(const moe_shape* shape);

/* Bytes of device workspace the named call needs (256-byte aligned start
 * required).  0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t kind);

/* Checks a shape; returns MOE_OK, MOE_ERR_INVALID_ARGUMENT or MOE_ERR_UNSUPPORTED. */
moe_status moe_check_shape(const moe_shape* shape);

/* Static string for a status code (never NULL). */
const char* moe_status_str(int32_t status);

/* ---- hot-path calls ---------------------------------------------------- */

/* Router scores, softmax, top-k and routing weights (ch. 36 §36.1-§36.2,
 * Algorithm 36.1 selection step; "MoE token routing" §2).
 *   x        [T,d]  dtype
 *   w_r      [E,d]  fp32;  b_r [E] fp32 or NULL
 *   topk_ids [T,P]  int32 out: rank order (descending fp32 score, lower id first on ties);
 *                   P = k, or 2k with shape->reroute (then the k next choices follow)
 *   topk_w   [T,P]  fp32 out: RENORM a = p_e / sum_{j in S} p_j (sums to 1);
 *                   SWITCH a = p_e (full softmax)
 *   status   [1]    int32 out: set to MOE_OK, or MOE_ERR_NONFINITE_LOGIT if any
 *                   score is NaN/Inf; such a token gets ids 0..k-1 and weights 0
 *                   so that later calls stay in bounds.  Read it after the
 *                   stream synchronises.
 *   ws              >= moe_workspace_bytes(shape, MOE_WS_ROUTE) bytes, starting with
 *                   the MOE_SYNC_BYTES sync words (zero before the first call on
 *                   this workspace; every call leaves them zero).  After them, bf16
 *                   activations: with T <= 16, nothing for E <= 8 and the fp32
 *                   partial scores of each 2048-wide K range for E > 8; with
 *                   T > 16, nothing for E <= 8, the bf16 split of w_r for E > 8,
 *                   plus fp32 partial scores when E > 64.  fp32 activations: the
 *                   [T,E] scores when E > 64. */
moe_status moe_route(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                     int32_t* topk_ids, float* topk_w, int32_t* status, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_route plus the router's probability mass per expert, the summable half of
 * the load-balance statistics (ch. 36 §36.4: merge probability sums and token
 * counts first, then form means over the chosen scope).
 *   prob_sum [E] fp32 out: sum over the T tokens of the full softmax p_e(x_t)
 *                          of the (biased) fp32 scores, in a fixed order; a token
 *                          with a non-finite score adds 0
 *   ws       >= moe_workspace_bytes(shape, MOE_WS_ROUTE_STATS) bytes: moe_route's
 *            workspace followed by the [T,E] fp32 probabilities
 * Other arguments as moe_route; same ids, weights and status. */
moe_status moe_route_stats(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                           int32_t* topk_ids, float* topk_w, int32_t* status, float* prob_sum, void* ws,
                           size_t ws_bytes, void* stream);

/* Load-balance and rejection statistics (ch. 36 §36.4 definitions of f_e and
 * p_bar_e and the auxiliary balance product, its worked example's rejection
 * rates; "The real cost of sparse expert models" rho_max):
 *   load     [E] int32 in: L_e from moe_dispatch
 *   stats    [MOE_STAT_COUNT] int32 in: from moe_dispatch
 *   prob_sum [E] fp32 in: from moe_route_stats
 *   out      [2E + MOE_BAL_COUNT] fp32 out: f_e = L_e / (T k) for e < E, then
 *            p_bar_e = prob_sum_e / T, then the MOE_BAL_* values (all 0 for T = 0)
 * One small kernel on stream; nothing is read back to the host. */
moe_status moe_balance(const moe_shape* shape, const int32_t* load, const int32_t* stats,
                       const float* prob_sum, float* out, void* stream);

/* Capacity-limited dispatch and load statistics (ch. 36 §36.3, Algorithm
 * 36.1 acceptance step and its invariants; "The real cost of sparse expert
 * models" equations for C_e, O and rho_max).
 *   x         [T,d]      dtype
 *   topk_ids  [T,P]      int32 in (values must lie in [0,E); each row distinct; with
 *                        reroute, next-choice records may be -1); P as in moe_route
 *   topk_w    [T,P]      fp32 in: the routing weights; read only with
 *                        shape->accept_by_gate (then required; else may be NULL)
 *   load      [E]        int32 out: requested load L_e
 *   offsets   [E+1]      int32 out: exclusive prefix sum of min(L_e, C)
 *   slot      [T,P]      int32 out: slot c within the expert (number of earlier
 *                        tokens that requested the same expert; with
 *                        accept_by_gate, of earlier accepted tokens), or -1 if rejected
 *   row_of    [T,P]      int32 out: offsets[e] + slot, or -1.  With reroute, the
 *                        slot and row of next choice j (column k + j) are set when
 *                        the j-th rejected selection of the token was served there
 *   src_token [max_rows] int32 out: token of each grouped row (rows >= A untouched)
 *   x_perm    [max_rows,d] dtype out: x_perm[row] = x[src_token[row]]; rows are
 *                        grouped by expert, token order inside each expert
 *   stats     [MOE_STAT_COUNT] int32 out (see the MOE_STAT_* indices)
 *   ws        >= moe_workspace_bytes(shape, MOE_WS_DISPATCH) bytes */
moe_status moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                        const float* topk_w,
                        int32_t* load, int32_t* offsets, int32_t* slot, int32_t* row_of,
                        int32_t* src_token, void* x_perm, int32_t* stats,
                        void* ws, size_t ws_bytes, void* stream);

/* Routed expert FFNs over the grouped rows ("MoE token routing" §3; ch. 36
 * §36.1 gated expert and Algorithm 36.1 expert step):
 *   h = SiLU(x_perm W_gate[e]^T) (*) (x_perm W_up[e]^T)   (rounded to dtype)
 *   H = h W_down[e]^T                                     (fp32)
 * for the rows [offsets[e], offsets[e+1]) of every expert e.
 *   x_perm  [max_rows,d] dtype;  offsets [E+1] int32 (non-decreasing, offsets[0]=0,
 *           offsets[E] <= moe_max_rows, and no expert holding more than min(T, C)
 *           rows — as moe_dispatch builds them, a token adding at most one row per
 *           expert and an expert accepting at most C; with min(T, C) <= 8 the calls
 *           run as grouped GEMVs sized by that bound, and an expert holding more
 *           rows gets its first min(T, C) rows computed and the rest set to NaN)
 *   w_gate, w_up [E,m,d] dtype;  w_down [E,d,m] dtype
 *   H       [max_rows,d] fp32 out (rows >= offsets[E] untouched)
 *   ws      >= moe_workspace_bytes(shape, MOE_WS_FFN) (holds h) */
moe_status moe_expert_ffn(const moe_shape* shape, const void* x_perm, const int32_t* offsets,
                          const void* w_gate, const void* w_up, const void* w_down, float* H,
                          void* ws, size_t ws_bytes, void* stream);

/* The first half of moe_expert_ffn alone: h [max_rows,m] (dtype) out.  ws as for
 * moe_expert_ffn (MOE_WS_FFN is large enough); small batches use part of it for
 * the fp32 gate/up partials of a K split. */
moe_status moe_expert_gemm1(const moe_shape* shape, const void* x_perm, const int32_t* offsets,
                            const void* w_gate, const void* w_up, void* h,
                            void* ws, size_t ws_bytes, void* stream);

/* The second half of moe_expert_ffn alone: H [max_rows,d] fp32 out from h.  ws as
 * for moe_expert_ffn (MOE_WS_FFN is large enough); a K split's extra fp32
 * partials live there and are added into H before the call's last kernel ends. */
moe_status moe_expert_gemm2(const moe_shape* shape, const void* h, const int32_t* offsets,
                            const void* w_down, float* H, void* ws, size_t ws_bytes, void* stream);

/* Shared expert on every token, unweighted (ch. 36 §36.6; "Sizzling MoE
 * skewer analogy" DeepSeek-V3 formula): s = SwiGLU(x) with
 *   s_gate, s_up [m_shared,d] dtype;  s_down [d,m_shared] dtype;  s [T,d] fp32 out.
 *   ws >= moe_workspace_bytes(shape, MOE_WS_SHARED).  Needs shape->m_shared > 0. */
moe_status moe_shared_ffn(const moe_shape* shape, const void* x, const void* s_gate,
                          const void* s_up, const void* s_down, float* s,
                          void* ws, size_t ws_bytes, void* stream);

/* Weighted combine back into token order (Algorithm 36.1 combine step;
 * "MoE token routing" §3):
 *   y[t] = shared_out[t] + sum_{r=0..k-1, row_of[t,r] >= 0} topk_w[t,r] * H[row_of[t,r]]
 * summed in rank order r = 0..k-1, in fp32.  With shape->renorm_survivors each
 * topk_w[t,r] is first divided by the sum (rank order) of the token's accepted
 * weights.
 *   H [max_rows,d] fp32;  row_of, topk_w [T,P] (P = k, or 2k with reroute: every
 *   record with a row is added, in column order);  shared_out [T,d] fp32 or NULL;
 *   y [T,d] fp32 out (fully overwritten). */
moe_status moe_combine(const moe_shape* shape, const float* H, const int32_t* row_of,
                       const float* topk_w, const float* shared_out, float* y, void* stream);

/* The whole layer: route -> dispatch -> expert FFN (+ shared) -> combine,
 * queued on `stream` with no host synchronisation.  s_gate/s_up/s_down may be
 * NULL only when shape->m_shared == 0.  Outputs as in the calls above;
 * every intermediate lives in ws (>= moe_workspace_bytes(shape, MOE_WS_FORWARD)).
 * topk_ids, topk_w and slot have P columns as in moe_route (2k with reroute).
 * The results equal those of the staged calls bit for bit, but the path may
 * differ: with bf16 activations the expert GEMMs read each grouped row in place
 * from x through the dispatch's row map (no x_perm copy; the E <= 8 router also
 * makes the dispatch's per-block counts), and with T <= 16 (bf16, E <= 256,
 * acceptance in token order) route and dispatch run as one workgroup.  The
 * shared expert runs on a second, default-priority stream of the device that the
 * call forks from `stream` with an event and joins before the combine, so it
 * overlaps the routed path; the call stays ordered on `stream` (and capturable).
 * The library creates that stream and its two events once per device. */
moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                       const void* w_gate, const void* w_up, const void* w_down,
                       const void* s_gate, const void* s_up, const void* s_down,
                       float* y, int32_t* topk_ids, float* topk_w, int32_t* load,
                       int32_t* slot, int32_t* stats, int32_t* status,
                       void* ws, size_t ws_bytes, void* stream);

/* Weight repacking, once per weight set and outside the forward: a batched
 * transpose dst[b][j][i] = src[b][i][j] (b < batch, i < rows, j < cols) of
 * elements of elem_bytes (2: bf16, 4: fp32), the bits copied unchanged.  It
 * turns weights kept in the pages' x W layout, in-features x out-features
 * ("LLM from scratch" ch. 36 §36.1; §36.8 notes that libraries store the
 * transpose), into this library's out x in layout:
 *   router W_r [d,E] fp32           batch 1, rows d,   cols E     -> w_r [E,d]
 *   W_gate, W_up [E,d,m] dtype      batch E, rows d,   cols m     -> [E,m,d]
 *   W_down [E,m,d] dtype            batch E, rows m,   cols d     -> [E,d,m]
 *   shared gate / up [d,m_shared]   batch 1, rows d,   cols m_shared
 *   shared down [m_shared,d]        batch 1, rows m_shared, cols d
 *   src, dst   device buffers of batch x rows x cols elements; they must not
 *              overlap (no in-place transpose); the caller owns both
 * Returns MOE_ERR_INVALID_ARGUMENT (launching nothing) for a null pointer with a
 * non-empty matrix, negative sizes, elem_bytes other than 2 or 4, or
 * overlapping buffers, and MOE_ERR_UNSUPPORTED for batch > 65535,
 * rows > 4194240 or more than INT64_MAX / 4 bytes in all.  Asynchronous on
 * `stream`. */
moe_status moe_pack_weights(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols,
                            int32_t elem_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and results as moe_forward (bit for bit), but the workspace is a
 * file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on
 * every device it runs on until the process ends, and the shared expert runs on
 * `stream` itself (no side stream or event is created).  No call allocates or
 * frees memory.  The first call on a device resolves the array's address on
 * that device (make it outside graph capture); later calls only launch.
 * Returns MOE_ERR_WORKSPACE_TOO_SMALL, launching nothing, when
 * moe_workspace_bytes(shape, MOE_WS_FORWARD) exceeds the array (64 MiB covers,
 * e.g., the Mixtral-shaped layer up to T = 512, the DeepSeek-V3-like layer up
 * to T = 64 and the Switch-shaped layer at T = 1024).  Every call on a device
 * shares that device's array, whose contents persist between calls: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  Other arguments and outputs as moe_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_r, const float* b_r,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const void* s_gate, const void* s_up, const void* s_down,
                               float* y, int32_t* topk_ids, float* topk_w, int32_t* load,
                               int32_t* slot, int32_t* stats, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
