// Router: scores, stable softmax, top-k with the lower-id tie rule, routing weights.
//
//   g[t,e] = sum_i x[t,i] w_r[e,i] + b_r[e]        ("LLM from scratch" ch. 36 §36.1;
//                                                  "MoE token routing" §2)
//   S_t    = k distinct ids, descending score, equal scores -> lower id
//                                                  (ch. 36 Algorithm 36.1 selection step)
//   a_te   = RENORM: softmax over the selected scores (equal to renormalising the
//            full softmax within S_t, "MoE token routing" §2; ch. 36 eq. (36.5))
//            SWITCH: the full-softmax probability p_te (ch. 36 §36.2)
//
// Score GEMM with bf16 activations: w_r is fp32, so it is first split into three
// bf16 planes (hi + mid + lo carries all 24 significand bits of each weight), and
// x * w_r is formed as three exact bf16 x bf16 products accumulated in fp32 on the
// MFMA units -- an fp32 dot product up to summation order.
//
// E <= 8 (bf16 activations, T > 16): one kernel; each workgroup splits w_r into
//   the planes itself, chunk by chunk, as ready-made MFMA operands in LDS (two
//   16-column tiles: hi | mid and lo | 0), its lanes load their 16 tokens'
//   activations straight into the MFMA operands, then it selects
//   (route_lds8_kernel).
// E <= 64: one fused kernel; 8 waves share 16 tokens, each wave takes one K
//   slice with all its loads in flight at once, the slices are summed in LDS in a
//   fixed order and the waves select.
// E > 64: the three planes stacked as a [3E (padded to a multiple of 8), d]
//   bf16 matrix make the scores one ungrouped GEMM on the expert-GEMM kernel
//   ([T, 3E] fp32 per K split, the K range split so that the work fills the
//   GPU); a selection kernel with one wave per token adds, per expert, the three
//   plane columns of every split in a fixed order.
// Selection: k rounds of a 64-bit (order-preserving score key, ~id) wave arg-max.
// Everything is deterministic: fixed summation orders; the only atomics are
// integer counts (the E <= 8 path's completion count and non-finite flag).
#include <algorithm>

#include "common.h"
#include "dispatch_block.h"

namespace {

constexpr int RT_TOK = 16;       // fused kernel: tokens per workgroup
constexpr int RT_WAVES = 8;       //               waves (K slices) per workgroup
constexpr int RT_THREADS = 64 * RT_WAVES;


__global__ void zero_i32_kernel(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Split 8 fp32 weights into three bf16 vectors whose sum reproduces them.
__device__ __forceinline__ void split3(const float4 w0, const float4 w1, uint4& H, uint4& M, uint4& L) {
    float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        h[j] = f32_to_bf16_bits(v[j]);
        float r1 = v[j] - bf16_bits_to_f32(h[j]);
        m[j] = f32_to_bf16_bits(r1);
        float r2 = r1 - bf16_bits_to_f32(m[j]);
        l[j] = f32_to_bf16_bits(r2);
    }
    H = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    M = {m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16)};
    L = {l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
}

// w3[p][e][i] = plane p (hi, mid, lo) of w_r[e][i]; 8 weights per thread.  The
// pad8 chunks after the three planes are zeroed (rows that round 3E up to a
// multiple of 8 for the score GEMM).  status (nullable): cleared here, ahead of
// the kernels that select.
__global__ __launch_bounds__(256) void split_router_kernel(const float* __restrict__ w_r, int64_t n8,
                                                           uint4* __restrict__ w3, int64_t pad8,
                                                           int32_t* __restrict__ status) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (status && i == 0) *status = MOE_OK;
    if (i < pad8) w3[3 * n8 + i] = uint4{0u, 0u, 0u, 0u};
    if (i >= n8) return;
    const float4* src = reinterpret_cast<const float4*>(w_r) + 2 * i;
    uint4 H, M, L;
    split3(src[0], src[1], H, M, L);
    w3[i] = H;
    w3[n8 + i] = M;
    w3[2 * n8 + i] = L;
}

// Rows of the score GEMM's weight matrix: the three planes of w_r, padded to a multiple of 8.
inline int score_cols(int E) { return (3 * E + 7) / 8 * 8; }

__device__ __forceinline__ floatx4_t mfma3(const bf16x8_t a, const uint4 H, const uint4 M, const uint4 L,
                                           floatx4_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(L), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(M), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(H), acc, 0, 0, 0);
    return acc;
}

// ---------------------------------------------------------------------------
// selection and weights for one token (called by a whole wave)
// ---------------------------------------------------------------------------
// b_r, topk_ids and topk_w may point to global memory or LDS.  cnt (nullable,
// LDS): cnt[e] += 1 for every selected expert id.  kout: records written per
// token, k or (rerouting) 2k: min(kout, E) rounds, the ones after the first k
// being the next choices, weighted with the selection's normalizer; records past
// E get id -1 and weight 0.
template <int EPL>
__device__ void select_token(const float* __restrict__ row, const float* __restrict__ b_r, int E, int k, int kout,
                             int mode, int64_t t, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                             int32_t* __restrict__ status, float* __restrict__ probs, int* cnt = nullptr) {
    const int lane = threadIdx.x % 64;
    float v[EPL];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        float g = -INFINITY;
        if (e < E) {
            g = row[e] + (b_r ? b_r[e] : 0.f);
            bad |= !isfinite(g);
        }
        v[j] = g;
    }
    if (__any(bad)) {
        if (lane < kout) {
            topk_ids[t * kout + lane] = lane < k ? lane : -1;
            topk_w[t * kout + lane] = 0.f;
            if (cnt && lane < k) atomicAdd(&cnt[lane], 1);
        }
        if (lane == 0) *status = MOE_ERR_NONFINITE_LOGIT;
        if (probs) {
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (lane + 64 * j < E) probs[t * E + lane + 64 * j] = 0.f;
        }
        return;
    }
    // rounds of a wave arg-max over (score key, lower id first).
    const int rounds = min(kout, E);
    uint32_t taken = 0;
    int my_e = -1;
    float my_g = 0.f;
    for (int s = 0; s < rounds; ++s) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u)) {
                const unsigned long long key =
                    ((unsigned long long)float_order_key(v[j]) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)e);
                best = key > best ? key : best;
            }
        }
        best = wave_max_u64(best);
        const int e_sel = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        if ((e_sel & 63) == lane) taken |= 1u << (e_sel >> 6);
        float g_sel = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j == e_sel) g_sel = v[j];
        g_sel = __shfl(g_sel, e_sel & 63, MOE_WAVE);
        if (lane == s) {
            my_e = e_sel;
            my_g = g_sel;
        }
    }
    const float g_top = __shfl(my_g, 0, MOE_WAVE);   // the largest score
    if (probs) {   // full softmax over the E scores, for the balance statistics
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j < E) z += expf(v[j] - g_top);
        z = wave_sum(z);
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j < E) probs[t * E + lane + 64 * j] = expf(v[j] - g_top) / z;
    }
    float wgt;
    if (mode == MOE_GATE_SWITCH) {
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j < E) z += expf(v[j] - g_top);
        z = wave_sum(z);
        wgt = expf(my_g - g_top) / z;
    } else {
        const float ez = lane < rounds ? expf(my_g - g_top) : 0.f;
        const float z = wave_sum(lane < k ? ez : 0.f);
        wgt = ez / z;
    }
    if (lane < kout) {
        topk_ids[t * kout + lane] = my_e;
        topk_w[t * kout + lane] = lane < rounds ? wgt : 0.f;
        if (cnt && lane < k) atomicAdd(&cnt[my_e], 1);
    }
}

// ---------------------------------------------------------------------------
// E <= 8, bf16 activations, T > 16: 16 tokens per workgroup, weight planes in LDS
// ---------------------------------------------------------------------------
//
// Each workgroup takes 16 tokens over the whole K, in chunks of 512.  Per chunk,
// the workgroup splits the chunk of w_r (fp32) into three exact bf16 planes
// (hi + mid + lo carries all 24 significand bits; the hardware
// round-to-nearest-even conversion) and stores them in LDS as the B operands of
// v_mfma_f32_16x16x32_bf16 for two 16-column tiles, [hi e0..7 | mid e0..7] and
// [lo e0..7 | 0].  Wave w of 8 runs K steps 2w, 2w+1 of every chunk; each lane
// loads its own A fragment (16 bytes of its token row per step) straight from
// memory; 2 MFMAs per step, fp32 accumulation (three exact products per
// element: an fp32 dot product up to summation order).  The loads of the next
// RL_DEPTH chunks are in flight while a chunk is computed, in chunk order, so
// the in-order completion of loads never makes a chunk wait for a later one;
// the planes are double-buffered and chunk c + 1 is staged while chunk c is
// multiplied, so one barrier per chunk suffices.  At the end a lane adds its hi
// column, the mid column one lane over and its lo column, the waves' sums are
// added in wave order, and one thread per token selects.
//
// The status word needs no clearing launch: a workgroup that finds a
// non-finite score raises a flag in the sync words.  Standalone, every
// workgroup then counts itself done, and the last one writes the status from
// the flag and puts both words back to zero (relaxed device-scope atomics; the
// flag's atomic completes before the count's is issued).  In the forward (the
// router also writing the dispatch's counts) the dispatch's placement kernel
// turns the flag into the status instead.
constexpr int RL_TOK = MOE_ROUTE_TOK;               // tokens per workgroup
constexpr int RL_KC = 512;                          // K elements per chunk
constexpr int RL_STEPS = RL_KC / 32;                // MFMA K steps per chunk
constexpr int RL_DEPTH = 4;                         // chunks of loads in flight
constexpr int RL_WAVES = 8;                         // K steps of a chunk split over the waves
constexpr int RL_THREADS = 64 * RL_WAVES;
constexpr int RL_WI = 8 * RL_STEPS * 4 / RL_THREADS;       // 8-weight items per thread and chunk
constexpr int RL_SPW = RL_STEPS / RL_WAVES;                 // K steps per wave and chunk

// LDS slot of B-operand entry (step s, lane' l) inside its 64-entry tile: l with
// its low three bits XORed by ((l >> 4) & 3) | ((s & 1) << 2).  A wave reading a
// tile (lane' = lane) still covers 8 distinct bank groups per 8 lanes (the XOR is
// constant over them), and a wave writing the planes of one expert (8 lanes = 4
// groups of 8 x 2 steps) does too: no bank conflicts either way.
__device__ __forceinline__ int rl_slot(int s, int l) { return l ^ (((l >> 4) & 3) | ((s & 1) << 2)); }

// Split 8 fp32 weights into three bf16 vectors whose sum reproduces them exactly
// (round to nearest even at each level).
__device__ __forceinline__ void split3_rne(const float4 w0, const float4 w1, uint4& H, uint4& M, uint4& L) {
    const float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        const float r0 = v[2 * j] - __uint_as_float(h[j] << 16);
        const float r1 = v[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u);
        m[j] = pack_bf16x2(r0, r1);
        const float s0 = r0 - __uint_as_float(m[j] << 16);
        const float s1 = r1 - __uint_as_float(m[j] & 0xffff0000u);
        l[j] = pack_bf16x2(s0, s1);
    }
    H = {h[0], h[1], h[2], h[3]};
    M = {m[0], m[1], m[2], m[3]};
    L = {l[0], l[1], l[2], l[3]};
}

// Selection for one token whose (at most 8) scores one thread holds, bias
// included (experts past E hold -inf): min(kout, E) rounds of an arg-max in
// ascending id order with a strict comparison (equal scores keep the lower id);
// the first k are the selection, the rest the next choices (reroute).  Weights:
// RENORM the softmax over the selected k (a next choice: its exponential over the
// same sum), SWITCH the full softmax.  A non-finite token gets ids 0..k-1 (then
// -1) and weights 0.  Branch-free over the experts (selects on order keys; an
// unavailable expert has key 0, below every score's).  Returns the selected
// experts as a bit mask.
__device__ __forceinline__ uint32_t select8_thread(const float (&v)[8], bool bad, int E, int k, int kout, int mode,
                                                   int64_t t, int32_t* __restrict__ topk_ids,
                                                   float* __restrict__ topk_w, float* __restrict__ probs) {
    const int rounds = min(kout, E);
    uint32_t key[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) key[e] = e < E ? float_order_key(v[e]) : 0u;
    uint32_t taken = 0, sel = 0;
    int ids[8];
    float gs[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        ids[r] = -1;
        gs[r] = 0.f;
        if (r < rounds) {
            int best = 0;
            uint32_t bkey = 0u;
            float bval = v[0];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t ke = ((taken >> e) & 1u) ? 0u : key[e];
                const bool better = ke > bkey;
                best = better ? e : best;
                bkey = better ? ke : bkey;
                bval = better ? v[e] : bval;
            }
            taken |= 1u << best;
            if (r < k) sel = taken;
            ids[r] = best;
            gs[r] = bval;
        }
    }
    const float g_top = gs[0];
    float zall = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < E) zall += expf(v[e] - g_top);
    float ex[8], zs = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        ex[r] = r < rounds ? expf(gs[r] - g_top) : 0.f;
        if (r < k) zs += ex[r];
    }
    const float z = mode == MOE_GATE_SWITCH ? zall : zs;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r < kout) {
            int id = r < rounds ? ids[r] : -1;
            float wt = r < rounds ? ex[r] / z : 0.f;
            if (bad) {
                id = r < k ? r : -1;
                wt = 0.f;
            }
            topk_ids[t * kout + r] = id;
            topk_w[t * kout + r] = wt;
        }
    }
    if (probs) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < E) probs[t * E + e] = bad ? 0.f : expf(v[e] - g_top) / zall;
    }
    return bad ? (1u << k) - 1u : sel;
}

// Wave 0 of a 16-token router workgroup, after the waves' partial scores are in
// red[wave][token * 8 + expert]: one lane per token adds them in wave order plus
// the bias and selects; the workgroup's per-expert selection counts go to hist
// (for the dispatch).  Non-finite scores raise the flag in the sync words.
// Without hist the workgroup then counts itself done (its atomic in flight during
// the selection), and the last workgroup to finish writes the status and puts the
// sync words back to zero (relaxed device-scope atomics; the flag's atomic
// completes before the count's is issued).  With hist the counting is skipped:
// the dispatch kernel that consumes the counts runs after this launch and turns
// the flag into the status (one atomic, off this kernel's critical path).
__device__ __forceinline__ void route8_select(const float (*red)[RL_TOK * 8], int64_t t0, int64_t T, int E, int k,
                                              int kout, int mode, const float* __restrict__ b_r,
                                              int32_t* __restrict__ sync, int32_t* __restrict__ topk_ids,
                                              float* __restrict__ topk_w, int32_t* __restrict__ status,
                                              float* __restrict__ probs, int32_t* __restrict__ hist) {
    const int lane = threadIdx.x % 64;
    const int r = lane;
    const int64_t t = t0 + r;
    const bool valid = r < RL_TOK && t < T;
    const int rr = min(r, RL_TOK - 1);
    float s[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float4 a = reinterpret_cast<const float4*>(red[0] + rr * 8)[h];
        s[4 * h] = a.x;
        s[4 * h + 1] = a.y;
        s[4 * h + 2] = a.z;
        s[4 * h + 3] = a.w;
    }
#pragma unroll
    for (int w = 1; w < RL_WAVES; ++w) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4 a = reinterpret_cast<const float4*>(red[w] + rr * 8)[h];
            s[4 * h] += a.x;
            s[4 * h + 1] += a.y;
            s[4 * h + 2] += a.z;
            s[4 * h + 3] += a.w;
        }
    }
    float v[8];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        v[e] = -INFINITY;
        if (e < E) {
            v[e] = s[e] + (b_r ? b_r[e] : 0.f);
            bad |= valid && !isfinite(v[e]);
        }
    }
    // with hist (the forward), the dispatch's placement kernel that reads the
    // counts writes the status from the flag: no workgroup here waits for an atomic
    const bool defer = hist != nullptr;
    if (__any(bad) && lane == 0) {
        atomicOr(&sync[1], 1);
        if (!defer) __builtin_amdgcn_s_waitcnt(0);   // the flag is in before this workgroup counts itself done
    }
    int done = 0;
    if (lane == 0 && !defer) done = atomicAdd(&sync[0], 1);
    uint32_t sel = 0;
    if (valid) sel = select8_thread(v, bad, E, k, kout, mode, t, topk_ids, topk_w, probs);
    if (hist) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int cnt = __popcll(__ballot((sel >> e) & 1u));
            if (e < E && lane == e) hist[(int64_t)blockIdx.x * E + e] = cnt;
        }
    }
    if (lane == 0 && !defer && done == (int)gridDim.x - 1) {   // the last workgroup
        *status = atomicExch(&sync[1], 0) ? MOE_ERR_NONFINITE_LOGIT : MOE_OK;
        atomicExch(&sync[0], 0);
    }
}

template <int NCT>   // chunks, fully unrolled (chunks past d are zero chunks)
__global__ __launch_bounds__(RL_THREADS) void route_lds8_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ b_r, int64_t T, int d,
    int E, int k, int kout, int mode, int32_t* __restrict__ sync, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ status, float* __restrict__ probs, int32_t* __restrict__ hist,
    int32_t* __restrict__ acc_stats) {
    __shared__ uint4 bs[2][RL_STEPS * 128];
    __shared__ __align__(16) float red[RL_WAVES][RL_TOK * 8];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int64_t t0 = (int64_t)blockIdx.x * RL_TOK;
    const int NC = (d + RL_KC - 1) / RL_KC;   // <= NCT
    if (acc_stats && blockIdx.x == 0 && tid < 2) acc_stats[tid] = 0;
    // the zero quarter of the second column tile (lanes 16 q + 8..15) never changes
    for (int i = tid; i < 2 * RL_STEPS * 32; i += RL_THREADS) {
        const int b = i / (RL_STEPS * 32), r = i % (RL_STEPS * 32), s = r / 32, z = r % 32;
        bs[b][s * 128 + 64 + rl_slot(s, 16 * (z / 8) + 8 + z % 8)] = uint4{0u, 0u, 0u, 0u};
    }
    const int lr = lane % 16, grp = lane / 16;
    // Loads of chunk c, every one unconditional from a clamped, valid address (a
    // chunk past the last repeats it, K past d reads the row's last 16 bytes and
    // is zeroed before use).  Activations go straight to the MFMA A operand: lane
    // (token lr, group grp) loads the 16 bytes at K offset 32 s + 8 grp of each of
    // its wave's steps s.  Weights: item it = tid + 512 j of 8 experts x 16 steps x
    // 4 groups of 8 (expert it / 64, step (it / 4) % 16, group it % 4), 32 bytes
    // each, split into the LDS planes by the whole workgroup.
    const uint16_t* xrow = x + min(t0 + lr, T - 1) * (int64_t)d;
    uint4 xr[RL_DEPTH][RL_SPW];
    float4 wr[RL_DEPTH][RL_WI][2];
    auto issue_x = [&](int slot, int c) {
        const int cc = min(c, NC - 1);
#pragma unroll
        for (int j = 0; j < RL_SPW; ++j) {
            const int kk = min(cc * RL_KC + 32 * (RL_SPW * wave + j) + 8 * grp, d - 8);
            xr[slot][j] = *reinterpret_cast<const uint4*>(xrow + kk);
        }
        // keep the loads in issue order: the in-order completion count then waits
        // for exactly the chunk in hand
        __builtin_amdgcn_sched_barrier(0);
    };
    auto issue_w = [&](int slot, int c) {
        const int cc = min(c, NC - 1);
#pragma unroll
        for (int j = 0; j < RL_WI; ++j) {
            const int it = tid + RL_THREADS * j;
            const int e = min(it / 64, E - 1);
            const int kk = min(cc * RL_KC + 32 * ((it / 4) % RL_STEPS) + 8 * (it % 4), d - 8);
            const float4* src = reinterpret_cast<const float4*>(w_r + (int64_t)e * d + kk);
            wr[slot][j][0] = src[0];
            wr[slot][j][1] = src[1];
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int u = 0; u < RL_DEPTH; ++u) {
        issue_w(u, u);
        issue_x(u, u);
    }
    // Chunk c's weights -> the planes of LDS buffer c & 1 (zero for experts >= E
    // and K past d); the freed ring slot takes the weights of chunk c + RL_DEPTH.
    auto stage = [&](int c) {
        const int u = c % RL_DEPTH, buf = c & 1;
#pragma unroll
        for (int j = 0; j < RL_WI; ++j) {
            const int it = tid + RL_THREADS * j;
            const int e = it / 64, s = (it / 4) % RL_STEPS, q = it % 4;
            uint4 H, M, Lo;   // split unconditionally, zeroed by a mask
            split3_rne(wr[u][j][0], wr[u][j][1], H, M, Lo);
            const uint32_t keep = e < E && c * RL_KC + 32 * s + 8 * q < d ? 0xffffffffu : 0u;
            uint4* b = &bs[buf][s * 128];
            b[rl_slot(s, 16 * q + e)] = uint4{H.x & keep, H.y & keep, H.z & keep, H.w & keep};
            b[rl_slot(s, 16 * q + e + 8)] = uint4{M.x & keep, M.y & keep, M.z & keep, M.w & keep};
            b[64 + rl_slot(s, 16 * q + e)] = uint4{Lo.x & keep, Lo.y & keep, Lo.z & keep, Lo.w & keep};
        }
        if (c + RL_DEPTH < NCT) issue_w(u, c + RL_DEPTH);
    };
    floatx4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // Software pipeline, one barrier per chunk: while chunk c's weight planes are
    // read from LDS and multiplied, chunk c + 1's are split and staged into the
    // other buffer (last read for chunk c - 1, before the previous barrier).
    // Straight-line code over the chunks (no loop back-edge, no branch on loaded
    // data), so the compiler's load counting waits for exactly the chunk in hand.
    stage(0);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const int u = c % RL_DEPTH, buf = c & 1;
        uint4 b0[RL_SPW], b1[RL_SPW];
#pragma unroll
        for (int j = 0; j < RL_SPW; ++j) {
            const int s = RL_SPW * wave + j;
            b0[j] = bs[buf][s * 128 + rl_slot(s, lane)];
            b1[j] = bs[buf][s * 128 + 64 + rl_slot(s, lane)];
        }
        if (c + 1 < NCT) stage(c + 1);
#pragma unroll
        for (int j = 0; j < RL_SPW; ++j) {
            const uint32_t keep = c * RL_KC + 32 * (RL_SPW * wave + j) + 8 * grp < d ? 0xffffffffu : 0u;
            const uint4 v = xr[u][j];
            const uint4 a = {v.x & keep, v.y & keep, v.z & keep, v.w & keep};
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b0[j]), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b1[j]), acc1, 0, 0, 0);
        }
        if (c + RL_DEPTH < NCT) issue_x(u, c + RL_DEPTH);
        if (c + 1 < NCT) __syncthreads();
    }
    // lane (lr, grp) holds column lr of both tiles for tokens 4 grp + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float mid = __shfl_xor(acc0[i], 8, MOE_WAVE);
        if (lr < 8) red[wave][(4 * grp + i) * 8 + lr] = (acc0[i] + mid) + acc1[i];
    }
    __syncthreads();
    if (wave == 0) route8_select(red, t0, T, E, k, kout, mode, b_r, sync, topk_ids, topk_w, status, probs, hist);
}

// ---------------------------------------------------------------------------
// E <= 64: fused scores + selection, 16 tokens per workgroup, 8 K slices
// ---------------------------------------------------------------------------

// Wave `wave` adds x[t0..t0+15] . w3[e] over its K slice for every expert column
// tile; results land in part[wave][16][Epad].  All loads of the slice are issued
// before the first MFMA.
template <int NT>
__device__ void scores_bf16_small(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w3, int64_t t0,
                                  int64_t T, int d, int E, float* part) {
    constexpr int KU = 8 / NT;                     // k-steps of 32 in flight (x + 3 planes per column tile)
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int row = lane % 16, grp = lane / 16;
    const int64_t t = t0 + row;
    const bool tok_ok = t < T;
    const uint16_t* xrow = x + (tok_ok ? t : 0) * (int64_t)d + grp * 8;
    const int64_t plane = (int64_t)E * d;
    const int kchunks = (d + 31) / 32;
    const int per = (kchunks + RT_WAVES - 1) / RT_WAVES;
    const int kbeg = wave * per * 32, kend = min(d, (wave + 1) * per * 32);

    floatx4_t acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kbeg; k0 < kend; k0 += 32 * KU) {
        uint4 av[KU], bw[KU][NT][3];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int kk = k0 + 32 * u + grp * 8;
            const bool k_ok = kk < kend;
            av[u] = (tok_ok && k_ok) ? *reinterpret_cast<const uint4*>(xrow + k0 + 32 * u) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int e = c * 16 + row;
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    bw[u][c][p] = (e < E && k_ok)
                                      ? *reinterpret_cast<const uint4*>(w3 + p * plane + (int64_t)e * d + kk)
                                      : uint4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int c = 0; c < NT; ++c)
                acc[c] = mfma3(as_bf16x8(av[u]), bw[u][c][0], bw[u][c][1], bw[u][c][2], acc[c]);
    }
    // lane holds expert column (lane % 16) of tile c, token rows 4*(lane/16) + i
    constexpr int Epad = NT * 16;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[(wave * RT_TOK + 4 * grp + i) * Epad + c * 16 + row] = acc[c][i];
}

// Scores with fp32 activations: plain fp32 fused multiply-add dot products.
__device__ void scores_f32(const float* __restrict__ x, const float* __restrict__ w_r, int64_t t0, int64_t T,
                           int d, int E, int ntok, float* lg) {
    for (int p = threadIdx.x; p < ntok * E; p += blockDim.x) {
        const int r = p / E, e = p % E;
        const int64_t t = t0 + r;
        float s = 0.f;
        if (t < T) {
            const float* xr = x + t * (int64_t)d;
            const float* wr = w_r + (int64_t)e * d;
            for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
        }
        lg[p] = s;
    }
}

template <bool BF16, int NT>
__global__ __launch_bounds__(RT_THREADS) void route_small_kernel(const void* __restrict__ xv,
                                                                 const float* __restrict__ w_r,
                                                                 const uint16_t* __restrict__ w3,
                                                                 const float* __restrict__ b_r, int64_t T, int d,
                                                                 int E, int k, int kout, int mode,
                                                                 int32_t* __restrict__ topk_ids,
                                                                 float* __restrict__ topk_w,
                                                                 int32_t* __restrict__ status,
                                                                 float* __restrict__ probs, int zero_status) {
    if (zero_status && threadIdx.x == 0) *status = MOE_OK;   // one-workgroup launch
    __shared__ float lg[RT_TOK * NT * 16];
    __shared__ float part[BF16 ? RT_WAVES * RT_TOK * NT * 16 : 1];
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;
    if (BF16) {
        scores_bf16_small<NT>(static_cast<const uint16_t*>(xv), w3, t0, T, d, E, part);
        __syncthreads();
        for (int p = threadIdx.x; p < RT_TOK * E; p += RT_THREADS) {
            const int r = p / E, e = p % E;
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < RT_WAVES; ++q) s += part[(q * RT_TOK + r) * NT * 16 + e];
            lg[p] = s;
        }
    } else {
        scores_f32(static_cast<const float*>(xv), w_r, t0, T, d, E, RT_TOK, lg);
    }
    __syncthreads();
    const int wave = threadIdx.x / 64;
    for (int r = wave; r < RT_TOK; r += RT_WAVES) {
        const int64_t t = t0 + r;
        if (t >= T) break;
        select_token<1>(lg + r * E, b_r, E, k, kout, mode, t, topk_ids, topk_w, status, probs);
    }
}

// ---------------------------------------------------------------------------
// E > 64: split-K score kernel + selection kernel
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void router_scores_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ w_r, int64_t T, int d,
                                                                int E, float* __restrict__ scores) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= T * E) return;
    const int64_t t = p / E;
    const int e = (int)(p % E);
    const float* xr = x + t * (int64_t)d;
    const float* wr = w_r + (int64_t)e * d;
    float s = 0.f;
    for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
    scores[p] = s;
}

// One wave per token: part holds KS blocks [T][NP]; the score of expert e is the
// sum over the blocks (in order) of its P plane columns p E + e, added lowest
// plane first; then selects.
template <int EPL>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ part, int KS, int P, int NP,
                                                           const float* __restrict__ b_r, int64_t T, int E, int k,
                                                           int kout, int mode, int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_w, int32_t* __restrict__ status,
                                                           float* __restrict__ probs, int zero_status) {
    __shared__ float rows[4][EPL * 64];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (zero_status) {   // one-workgroup launch: clear the status word first
        if (threadIdx.x == 0) *status = MOE_OK;
        __syncthreads();
    }
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    // s_e = sum over K splits q (in order) of the planes pl = P-1 .. 0 (in that
    // order); the loads of four splits are issued together, then added in order
    float sum[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) sum[j] = 0.f;
    for (int q0 = 0; q0 < KS; q0 += 4) {
        float v[EPL][4][3];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
#pragma unroll
                for (int pl = 0; pl < 3; ++pl)
                    v[j][qq][pl] = (e < E && q0 + qq < KS && pl < P)
                                       ? part[((int64_t)(q0 + qq) * T + t) * NP + pl * E + e]
                                       : 0.f;
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                if (q0 + qq < KS)
#pragma unroll
                    for (int pl = 2; pl >= 0; --pl)
                        if (pl < P) sum[j] += v[j][qq][pl];
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (e < E) rows[wave][e] = sum[j];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    select_token<EPL>(rows[wave], b_r, E, k, kout, mode, t, topk_ids, topk_w, status, probs);
}

// ---------------------------------------------------------------------------
// small batches (T <= DOT_TMAX), bf16 activations, E > 8: direct fp32 dot products
// ---------------------------------------------------------------------------
//
// Workgroup (g, q) owns experts [DOT_EW g, DOT_EW g + DOT_EW) for all T tokens
// over the K range [2048 q, 2048 q + 2048), so w_r is read once over the grid and
// every load of a workgroup is in flight at once.  Thread j multiplies the 8-wide
// K chunk 2048 q + 8 j of its experts' fp32 weights with every token's exactly
// upcast activations (fp32 FMAs), then the (token, expert) sums are reduced over
// the wave with a fixed xor pattern and over the 4 waves in order:
// part[(q T + t) E + e], no bias (the selection adds the K ranges in order, then
// the bias).  An fp32 dot product up to summation order, like the plane split.
constexpr int DOT_TMAX = 16;
constexpr int DOT_EW = 2;

__global__ __launch_bounds__(256) void route_dot_kernel(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ w_r, int64_t T, int d, int E,
                                                        float* __restrict__ part) {
    __shared__ float red[4][DOT_TMAX * DOT_EW];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int e0 = blockIdx.x * DOT_EW;
    const int q = blockIdx.y;
    float acc[DOT_TMAX][DOT_EW];
#pragma unroll
    for (int t = 0; t < DOT_TMAX; ++t)
#pragma unroll
        for (int j = 0; j < DOT_EW; ++j) acc[t][j] = 0.f;
    const int c = q * 2048 + 8 * tid;
    if (c < d) {   // d % 8 == 0: a chunk is wholly in
        float w[DOT_EW][8];
#pragma unroll
        for (int j = 0; j < DOT_EW; ++j) {
            const int e = min(e0 + j, E - 1);
            const float4 lo = *reinterpret_cast<const float4*>(w_r + (int64_t)e * d + c);
            const float4 hi = *reinterpret_cast<const float4*>(w_r + (int64_t)e * d + c + 4);
            w[j][0] = lo.x; w[j][1] = lo.y; w[j][2] = lo.z; w[j][3] = lo.w;
            w[j][4] = hi.x; w[j][5] = hi.y; w[j][6] = hi.z; w[j][7] = hi.w;
        }
#pragma unroll
        for (int t = 0; t < DOT_TMAX; ++t) {
            if (t < T) {
                const uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)t * d + c);
                const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = __uint_as_float(xw[i] << 16), x1 = __uint_as_float(xw[i] & 0xffff0000u);
#pragma unroll
                    for (int j = 0; j < DOT_EW; ++j) {
                        acc[t][j] = fmaf(x0, w[j][2 * i], acc[t][j]);
                        acc[t][j] = fmaf(x1, w[j][2 * i + 1], acc[t][j]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < DOT_TMAX; ++t)
#pragma unroll
        for (int j = 0; j < DOT_EW; ++j) {
            float v = acc[t][j];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
            if (lane == 0) red[wave][t * DOT_EW + j] = v;
        }
    __syncthreads();
    if (tid < DOT_TMAX * DOT_EW) {
        const int t = tid / DOT_EW, j = tid % DOT_EW, e = e0 + j;
        if (t < T && e < E)
            part[((int64_t)q * T + t) * E + e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// v[e], e < 8, summed over the 16 lanes of a row; lane l ends with expert l & 7.
// Pairings: l <-> 7 - l within 8 lanes (row half mirror), l <-> l ^ 2, l <-> l ^ 1
// (quad permutes), then l <-> l + 8 mod 16 (row rotate by 8).
__device__ __forceinline__ float reduce_row8(const float (&v)[8]) {
    const int lane = threadIdx.x % 64;
    const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
    float u[4], w2[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // keep experts 4 b2 + 0..3
        const float keep = b2 ? v[4 + i] : v[i], give = b2 ? v[i] : v[4 + i];
        u[i] = keep + dpp_mov<0x141>(give);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {   // keep experts 4 b2 + 2 b1 + 0..1
        const float keep = b1 ? u[2 + i] : u[i], give = b1 ? u[i] : u[2 + i];
        w2[i] = keep + dpp_mov<0x4E>(give);
    }
    float r = (b0 ? w2[1] : w2[0]) + dpp_mov<0xB1>(b0 ? w2[0] : w2[1]);
    return r + dpp_mov<0x128>(r);
}

// ---------------------------------------------------------------------------
// T <= 16, bf16, E <= 256: the front of the layer in one workgroup
// ---------------------------------------------------------------------------
//
// One workgroup of 1024 threads clears the status word, forms the scores, selects
// (wave t takes token t) and, with DISPATCH, dispatches the block (the same
// integer results as the dispatch kernels) and copies every accepted row to its
// grouped position -- one launch where the large-batch path takes four or more.
// Scores for E <= 8: fp32 FMA dot products.  Thread j holds the K chunk [4 j,
// 4 j + 4) of every K range of 4096 for all E weight rows (fp32, as given) and
// per token reduces its 8 expert partials over each 16-lane row with DPP moves;
// the rows' sums are accumulated in LDS over the K ranges in order, then added
// over the rows in order.  E > 8: the sum, in split order, of route_dot_kernel's
// partials.
constexpr int FS_TOK = DOT_TMAX;
constexpr int FS_EMAX = 256;
constexpr int FS_THREADS = 1024;
constexpr int FS_WAVES = FS_THREADS / 64;
constexpr int FS_KR = 4 * FS_THREADS;   // K elements per range

template <int EPL, bool DISPATCH>
__global__ __launch_bounds__(FS_THREADS) void front_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ dpart, int KS,
    const float* __restrict__ b_r, int64_t T, int d, int E, int k, int kout, int C, int mode,
    int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ status, float* __restrict__ probs, int32_t* __restrict__ load,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ row_of,
    int32_t* __restrict__ src_token, uint4* __restrict__ x_perm, int32_t* __restrict__ stats,
    int32_t* __restrict__ tprefix, int tile_rows) {
    __shared__ float lg[FS_TOK * FS_EMAX];
    __shared__ float part[64 * FS_TOK * 8];   // (16-lane row, token, expert)
    __shared__ float s_bias[FS_EMAX];
    __shared__ unsigned long long masks[DISPATCH ? 4 * FS_EMAX : 1];
    __shared__ int s_off[DISPATCH ? FS_EMAX : 1];
    __shared__ int s_ids[DISPATCH ? FS_TOK * 32 : 1];
    __shared__ float s_w[DISPATCH ? FS_TOK * 32 : 1];
    __shared__ int s_row[DISPATCH ? FS_TOK * 32 : 1];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    if (tid == 0) *status = MOE_OK;   // before the barriers that precede every selection
    const float bias = (tid < E && b_r) ? b_r[tid] : 0.f;   // to LDS before the selection's barrier
    if (E <= 8) {
        const int row = tid / 16;   // 16-lane row, 0..63
        for (int kr = 0; kr * FS_KR < d; ++kr) {
            const int c = kr * FS_KR + 4 * tid;
            const bool c_ok = c < d;   // d % 8 == 0: a chunk of 4 is wholly in or out
            const int cc = c_ok ? c : d - 4;
            // all loads unconditional (clamped addresses), invalid values zeroed afterwards
            float w[8][4];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float4 v = *reinterpret_cast<const float4*>(w_r + (int64_t)min(e, E - 1) * d + cc);
                const bool ok = c_ok && e < E;
                w[e][0] = ok ? v.x : 0.f;
                w[e][1] = ok ? v.y : 0.f;
                w[e][2] = ok ? v.z : 0.f;
                w[e][3] = ok ? v.w : 0.f;
            }
            for (int t0 = 0; t0 < T; t0 += 8) {
                uint2 xv[8];   // the next eight tokens
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    xv[i] = *reinterpret_cast<const uint2*>(x + min((int64_t)(t0 + i), T - 1) * d + cc);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int t = t0 + i;
                    if (t >= T) break;
                    // a chunk past d adds 0 (not 0 * x, which may be NaN)
                    const float xf[4] = {c_ok ? __uint_as_float(xv[i].x << 16) : 0.f,
                                         c_ok ? __uint_as_float(xv[i].x & 0xffff0000u) : 0.f,
                                         c_ok ? __uint_as_float(xv[i].y << 16) : 0.f,
                                         c_ok ? __uint_as_float(xv[i].y & 0xffff0000u) : 0.f};
                    float acc[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float sum = 0.f;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) sum = fmaf(xf[jj], w[e][jj], sum);
                        acc[e] = sum;
                    }
                    const float sum = reduce_row8(acc);
                    if ((lane & 15) < 8) {
                        float* dst = &part[(row * FS_TOK + t) * 8 + (lane & 7)];
                        *dst = kr ? *dst + sum : sum;
                    }
                }
            }
        }
        __syncthreads();
        if (tid < FS_TOK * 8) {
            const int t = tid / 8, e = tid % 8;
            if (t < T && e < E) {
                float sc = 0.f;
#pragma unroll 16
                for (int r = 0; r < 64; ++r) sc += part[(r * FS_TOK + t) * 8 + e];
                lg[t * E + e] = sc;
            }
        }
    } else {
        for (int p = tid; p < T * E; p += FS_THREADS) {
            float sc = 0.f;
            for (int q0 = 0; q0 < KS; q0 += 8) {   // eight splits' loads in flight, added in order
                float v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = dpart[(int64_t)min(q0 + q, KS - 1) * T * E + p];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (q0 + q < KS) sc += v[q];
            }
            lg[p] = sc;
        }
    }
    if (tid < E) s_bias[tid] = bias;
    __syncthreads();
    // with DISPATCH the ids and weights go to LDS first and to memory at the end, so
    // no barrier below waits for their stores
    if (wave < T)
        select_token<EPL>(lg + wave * E, s_bias, E, k, DISPATCH ? k : kout, mode, wave, DISPATCH ? s_ids : topk_ids,
                          DISPATCH ? s_w : topk_w, status, probs);
    if (!DISPATCH) return;
    __syncthreads();
    dispatch_one_block(s_ids, T, k, E, C, load, offsets, stats, tprefix, tile_rows, slot, row_of, src_token, masks,
                       s_off, s_row);
    for (int p = tid; p < T * k; p += FS_THREADS) {
        topk_ids[p] = s_ids[p];
        topk_w[p] = s_w[p];
    }
    // copy every accepted row x[t] -> x_perm[row]: one wave per path, 4 x 16 B per lane in flight
    if (!x_perm) return;
    const int64_t vpr = d / 8;   // 16-byte vectors per bf16 row (d % 8 == 0)
    const uint4* xv4 = reinterpret_cast<const uint4*>(x);
    for (int p = wave; p < T * k; p += FS_WAVES) {
        const int row = s_row[p];
        if (row < 0) continue;
        const uint4* src = xv4 + (int64_t)(p / k) * vpr;
        uint4* dst = x_perm + (int64_t)row * vpr;
        for (int64_t c0 = lane; c0 < vpr; c0 += 4 * 64) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = src[min(c0 + 64 * u, vpr - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (c0 + 64 * u < vpr) dst[c0 + 64 * u] = v[u];
        }
    }
}

template <int EPL>
void launch_select(const moe_dims& s, const float* part, int KS, int P, int NP, const float* b_r, int32_t* ids,
                   float* w, int32_t* status, float* probs, hipStream_t st) {
    const unsigned grid = (unsigned)((s.T + 3) / 4);
    hipLaunchKernelGGL((route_select_kernel<EPL>), dim3(grid), dim3(256), 0, st, part, KS, P, NP, b_r, s.T, s.E, s.k,
                       moe_paths(s), s.gate_mode, ids, w, status, probs, grid == 1 ? 1 : 0);
}

// prob_sum[e] = sum over t of probs[t E + e]: 16 waves per 64 experts, wave w
// sums a contiguous sixteenth of the tokens (16 interleaved partial sums per
// lane, so 16 loads are in flight, added pairwise at the end), then the waves'
// sums are added in wave order.  Fixed order.
__global__ __launch_bounds__(1024) void prob_column_sum_kernel(const float* __restrict__ probs, int64_t T, int E,
                                                               float* __restrict__ prob_sum) {
    constexpr int NA = 16;
    __shared__ float ws[16][64];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int e = blockIdx.x * 64 + lane;
    const int64_t per = (T + 15) / 16;
    const int64_t t0 = min((int64_t)wave * per, T), t1 = min(t0 + per, T);
    float a[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) a[i] = 0.f;
    if (e < E) {
        int64_t t = t0;
        for (; t + NA <= t1; t += NA) {
#pragma unroll
            for (int i = 0; i < NA; ++i) a[i] += probs[(t + i) * E + e];
        }
#pragma unroll
        for (int i = 0; i < NA; ++i)
            if (t + i < t1) a[i] += probs[(t + i) * E + e];
    }
#pragma unroll
    for (int w = NA / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) a[i] += a[i + w];
    ws[wave][lane] = a[0];
    __syncthreads();
    if (wave == 0 && e < E) {
        float sum = 0.f;
        for (int w = 0; w < 16; ++w) sum += ws[w][lane];
        prob_sum[e] = sum;
    }
}

}  // namespace

namespace moe_kernels {

// route_lds8_kernel serves bf16 layers with E <= 8 and T > 16.
bool route_lds8_ok(const moe_dims& s) {
    return s.dtype == MOE_BF16 && s.E <= 8 && s.T > DOT_TMAX && s.d <= 32 * RL_KC;
}

size_t route_ws_bytes(const moe_dims& s) {
    if (s.dtype != MOE_BF16) return s.E > 64 ? (size_t)s.T * s.E * sizeof(float) : 0;
    if (s.T <= DOT_TMAX)   // front_small_kernel (E <= 8), else route_dot_kernel's partials
        return s.E <= 8 ? 0 : (size_t)((s.d + 2047) / 2048) * s.T * s.E * sizeof(float);
    if (route_lds8_ok(s)) return 0;   // the sync words only
    const int N3 = score_cols(s.E);
    size_t planes = ((size_t)N3 * s.d * 2 + 255) & ~(size_t)255;
    if (s.E <= 64) return planes;
    return planes + (size_t)scores_splits(s.T, N3, s.d) * s.T * N3 * sizeof(float);
}

bool front_fused_ok(const moe_dims& s) {
    return s.dtype == MOE_BF16 && s.T > 0 && s.T <= FS_TOK && s.E <= FS_EMAX && !s.accept_by_gate && !s.reroute;
}

namespace {

// T <= 16, bf16, E <= 256: route_dot_kernel (E > 8), then front_small_kernel.
template <bool DISPATCH>
hipError_t launch_front_small(const moe_dims& s, const void* x, const float* w_r, const float* b_r,
                              int32_t* topk_ids, float* topk_w, int32_t* status, float* probs, void* ws,
                              hipStream_t st, int32_t* load, int32_t* offsets, int32_t* slot, int32_t* row_of,
                              int32_t* src_token, void* x_perm, int32_t* stats, int32_t* tprefix, int tile_rows) {
    const float* dpart = nullptr;
    int KS = 0;
    if (s.E > 8) {
        KS = (s.d + 2047) / 2048;
        hipLaunchKernelGGL(route_dot_kernel, dim3((unsigned)((s.E + DOT_EW - 1) / DOT_EW), (unsigned)KS), dim3(256), 0,
                           st, static_cast<const uint16_t*>(x), w_r, s.T, s.d, s.E, static_cast<float*>(ws));
        dpart = static_cast<const float*>(ws);
    }
#define MOE_FRONT(EPLV)                                                                                         \
    hipLaunchKernelGGL((front_small_kernel<EPLV, DISPATCH>), dim3(1), dim3(FS_THREADS), 0, st,                 \
                       static_cast<const uint16_t*>(x), w_r, dpart, KS, b_r, s.T, s.d, s.E, s.k, moe_paths(s), s.C, \
                       s.gate_mode,                                                                           \
                       topk_ids, topk_w, status, probs, load, offsets, slot, row_of, src_token,                \
                       static_cast<uint4*>(x_perm), stats, tprefix, tile_rows)
    if (s.E <= 64) MOE_FRONT(1);
    else if (s.E <= 128) MOE_FRONT(2);
    else MOE_FRONT(4);
#undef MOE_FRONT
    return hipGetLastError();
}

}  // namespace

hipError_t launch_front(const moe_dims& s, const void* x, const float* w_r, const float* b_r, int32_t* topk_ids,
                        float* topk_w, int32_t* status, void* ws, hipStream_t st, int32_t* load, int32_t* offsets,
                        int32_t* slot, int32_t* row_of, int32_t* src_token, void* x_perm, int32_t* stats,
                        int32_t* tprefix, int tile_rows) {
    return launch_front_small<true>(s, x, w_r, b_r, topk_ids, topk_w, status, nullptr, ws, st, load, offsets, slot,
                                    row_of, src_token, x_perm, stats, tprefix, tile_rows);
}

hipError_t launch_route(const moe_dims& s, const void* x, const float* w_r, const float* b_r, int32_t* topk_ids,
                        float* topk_w, int32_t* status, void* ws, int32_t* sync, hipStream_t st, float* probs,
                        int32_t* hist, bool* hist_done, int32_t* acc_stats) {
    if (s.T == 0) {
        hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, st, status, 1);
        return hipGetLastError();
    }
    if (s.dtype == MOE_BF16 && s.T <= FS_TOK && s.E <= FS_EMAX)
        return launch_front_small<false>(s, x, w_r, b_r, topk_ids, topk_w, status, probs, ws, st, nullptr, nullptr,
                                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0);
    if (route_lds8_ok(s)) {
        const unsigned grid = (unsigned)((s.T + RL_TOK - 1) / RL_TOK);
        const int NC = (s.d + RL_KC - 1) / RL_KC;
#define MOE_LDS8(NCV)                                                                                           \
    hipLaunchKernelGGL((route_lds8_kernel<NCV>), dim3(grid), dim3(RL_THREADS), 0, st,                            \
                       static_cast<const uint16_t*>(x), w_r, b_r, s.T, s.d, s.E, s.k, moe_paths(s), s.gate_mode, \
                       sync, topk_ids, topk_w, status, probs, hist, hist ? acc_stats : nullptr)
        if (NC <= 1) MOE_LDS8(1);
        else if (NC <= 2) MOE_LDS8(2);
        else if (NC <= 4) MOE_LDS8(4);
        else if (NC <= 8) MOE_LDS8(8);
        else if (NC <= 16) MOE_LDS8(16);
        else MOE_LDS8(32);
#undef MOE_LDS8
        const hipError_t e = hipGetLastError();
        if (e == hipSuccess && hist && hist_done) *hist_done = true;
        return e;
    }
    // The status word is cleared before any selection may set it: by the plane split
    // (bf16), by the selecting kernel itself when that is a single workgroup, else by
    // a kernel of its own.
    const bool dot = s.dtype == MOE_BF16 && s.T <= DOT_TMAX;   // here E > 256
    // tokens per selecting workgroup
    const int64_t sel_tokens = dot || s.E > 64 ? 4 : RT_TOK;
    const bool self_zero = s.T <= sel_tokens;
    const bool split = s.dtype == MOE_BF16 && !dot;   // the plane split runs first and clears it
    if (!self_zero && !split) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, st, status, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dot) {
        float* dpart = static_cast<float*>(ws);
        const int KS = (s.d + 2047) / 2048;
        hipLaunchKernelGGL(route_dot_kernel, dim3((unsigned)((s.E + DOT_EW - 1) / DOT_EW), (unsigned)KS), dim3(256), 0,
                           st, static_cast<const uint16_t*>(x), w_r, s.T, s.d, s.E, dpart);
        if (s.E <= 128) launch_select<2>(s, dpart, KS, 1, s.E, b_r, topk_ids, topk_w, status, probs, st);
        else if (s.E <= 256) launch_select<4>(s, dpart, KS, 1, s.E, b_r, topk_ids, topk_w, status, probs, st);
        else if (s.E <= 512) launch_select<8>(s, dpart, KS, 1, s.E, b_r, topk_ids, topk_w, status, probs, st);
        else launch_select<16>(s, dpart, KS, 1, s.E, b_r, topk_ids, topk_w, status, probs, st);
        return hipGetLastError();
    }
    uint16_t* w3 = static_cast<uint16_t*>(ws);
    if (s.dtype == MOE_BF16) {
        const int64_t n8 = (int64_t)s.E * s.d / 8;
        const int64_t pad8 = s.E > 64 ? (int64_t)(score_cols(s.E) - 3 * s.E) * s.d / 8 : 0;
        hipLaunchKernelGGL(split_router_kernel, dim3((unsigned)((std::max(n8, pad8) + 255) / 256)), dim3(256), 0, st,
                           w_r, n8, reinterpret_cast<uint4*>(w3), pad8, status);
    }
    if (s.E <= 64) {
        const unsigned grid = (unsigned)((s.T + RT_TOK - 1) / RT_TOK);
        const int NT = (s.E + 15) / 16;
#define MOE_SMALL(NTV)                                                                                          \
    do {                                                                                                       \
        if (s.dtype == MOE_BF16)                                                                               \
            hipLaunchKernelGGL((route_small_kernel<true, NTV>), dim3(grid), dim3(RT_THREADS), 0, st, x, w_r, w3, \
                               b_r, s.T, s.d, s.E, s.k, moe_paths(s), s.gate_mode, topk_ids, topk_w, status,  \
                               probs, self_zero ? 1 : 0);                                                     \
        else                                                                                                   \
            hipLaunchKernelGGL((route_small_kernel<false, NTV>), dim3(grid), dim3(RT_THREADS), 0, st, x, w_r, w3, \
                               b_r, s.T, s.d, s.E, s.k, moe_paths(s), s.gate_mode, topk_ids, topk_w, status,  \
                               probs, self_zero ? 1 : 0);                                                     \
    } while (0)
        if (NT == 1) MOE_SMALL(1);
        else if (NT == 2) MOE_SMALL(2);
        else MOE_SMALL(4);
#undef MOE_SMALL
        return hipGetLastError();
    }
    // E > 64: scores as one ungrouped GEMM (bf16: x against the three planes, [T, 3E]
    // padded to N3 columns, K split over KS blocks; fp32: plain dot products)
    float* part;
    int KS = 1, P = 1, NP = s.E;
    if (s.dtype == MOE_BF16) {
        const int N3 = score_cols(s.E);
        part = reinterpret_cast<float*>(static_cast<char*>(ws) + (((size_t)N3 * s.d * 2 + 255) & ~(size_t)255));
        KS = scores_splits(s.T, N3, s.d);
        P = 3;
        NP = N3;
        e = launch_scores_gemm(x, w3, s.T, N3, s.d, part, st);
        if (e != hipSuccess) return e;
    } else {
        part = static_cast<float*>(ws);
        const unsigned grid = (unsigned)((s.T * s.E + 255) / 256);
        hipLaunchKernelGGL(router_scores_f32_kernel, dim3(grid), dim3(256), 0, st, static_cast<const float*>(x), w_r,
                           s.T, s.d, s.E, part);
    }
    if (s.E <= 128) launch_select<2>(s, part, KS, P, NP, b_r, topk_ids, topk_w, status, probs, st);
    else if (s.E <= 256) launch_select<4>(s, part, KS, P, NP, b_r, topk_ids, topk_w, status, probs, st);
    else if (s.E <= 512) launch_select<8>(s, part, KS, P, NP, b_r, topk_ids, topk_w, status, probs, st);
    else launch_select<16>(s, part, KS, P, NP, b_r, topk_ids, topk_w, status, probs, st);
    return hipGetLastError();
}

hipError_t launch_prob_sum(const moe_dims& s, const float* probs, float* prob_sum, hipStream_t st) {
    hipLaunchKernelGGL(prob_column_sum_kernel, dim3((unsigned)((s.E + 63) / 64)), dim3(1024), 0, st, probs, s.T, s.E,
                       prob_sum);
    return hipGetLastError();
}

}  // namespace moe_kernels
