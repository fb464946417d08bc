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
// One workgroup (4 waves) owns 16 tokens.  With bf16 activations the score GEMM
// runs on the bf16 MFMA units: w_r is fp32, so each 8-wide k-slice of w_r is split
// on the fly into three bf16 parts (hi + mid + lo carries all 24 significand bits)
// and x * w_r is formed as three exact bf16 x bf16 products accumulated in fp32.
// The 16 x E fp32 score tile is then reduced in LDS and every wave selects the
// top-k of its tokens with 64-bit (score-key, ~id) wave arg-max reductions.
#include "common.h"

namespace {

constexpr int RT_TOK = 16;
constexpr int RT_THREADS = 256;

__global__ void zero_i32_kernel(int32_t* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Split 8 fp32 weights into three bf16 vectors whose sum reproduces them.
__device__ __forceinline__ void split3(const float4 w0, const float4 w1, bf16x8_t& hi, bf16x8_t& mid,
                                       bf16x8_t& lo) {
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
    uint4 H = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    uint4 M = {m[0] | (m[1] << 16), m[2] | (m[3] << 16), m[4] | (m[5] << 16), m[6] | (m[7] << 16)};
    uint4 L = {l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
    hi = as_bf16x8(H);
    mid = as_bf16x8(M);
    lo = as_bf16x8(L);
}

// Scores of 16 tokens x E experts into lg[16][E] (bf16 x, MFMA 16x16x32).
template <int MAXT>
__device__ void scores_bf16_mfma(const uint16_t* __restrict__ x, const float* __restrict__ w_r, int64_t t0,
                                 int64_t T, int d, int E, float* lg, float* part) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int NT = (E + 15) / 16;
    const int CG = NT < 4 ? NT : 4;
    const int KS = 4 / CG;
    const int cg = wave % CG, ks = wave / CG;
    const int kchunks = (d + 31) / 32;
    const int per = (kchunks + KS - 1) / KS;
    const int kbeg = ks * per * 32;
    const int kend = min(d, (ks + 1) * per * 32);
    const bool active = ks < KS;

    floatx4_t acc[MAXT];
#pragma unroll
    for (int j = 0; j < MAXT; ++j) acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int row = lane % 16, grp = lane / 16;
    const int64_t t = t0 + row;
    const bool tok_ok = t < T;
    const uint16_t* xrow = x + (tok_ok ? t : 0) * (int64_t)d;

    if (active) {
        for (int k0 = kbeg; k0 < kend; k0 += 32) {
            const int kk = k0 + grp * 8;
            const bool k_ok = kk < kend;
            uint4 av = {0u, 0u, 0u, 0u};
            if (tok_ok && k_ok) av = *reinterpret_cast<const uint4*>(xrow + kk);
            const bf16x8_t a = as_bf16x8(av);
#pragma unroll
            for (int j = 0; j < MAXT; ++j) {
                const int ct = cg + j * CG;
                if (ct < NT) {
                    const int e = ct * 16 + row;
                    float4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
                    if (e < E && k_ok) {
                        const float4* wp = reinterpret_cast<const float4*>(w_r + (int64_t)e * d + kk);
                        w0 = wp[0];
                        w1 = wp[1];
                    }
                    bf16x8_t hi, mid, lo;
                    split3(w0, w1, hi, mid, lo);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, mid, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc[j], 0, 0, 0);
                }
            }
        }
    }
    // Accumulator layout: lane holds column (lane % 16), rows 4*(lane/16) + i.
    const int Epad = NT * 16;
    if (active) {
#pragma unroll
        for (int j = 0; j < MAXT; ++j) {
            const int ct = cg + j * CG;
            if (ct < NT) {
                const int e = ct * 16 + (lane % 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * (lane / 16) + i;
                    if (KS == 1) {
                        if (e < E) lg[r * E + e] = acc[j][i];
                    } else {
                        part[(ks * RT_TOK + r) * Epad + e] = acc[j][i];
                    }
                }
            }
        }
    }
    if (KS > 1) {
        __syncthreads();
        for (int p = threadIdx.x; p < RT_TOK * E; p += RT_THREADS) {
            const int r = p / E, e = p % E;
            float s = 0.f;
            for (int q = 0; q < KS; ++q) s += part[(q * RT_TOK + r) * Epad + e];
            lg[p] = s;
        }
    }
}

// Scores with fp32 activations: plain fp32 fused multiply-add dot products.
__device__ void scores_f32(const float* __restrict__ x, const float* __restrict__ w_r, int64_t t0, int64_t T,
                           int d, int E, float* lg) {
    for (int p = threadIdx.x; p < RT_TOK * E; p += RT_THREADS) {
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

template <int EPL, bool BF16>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(const void* __restrict__ xv, const float* __restrict__ w_r,
                                                           const float* __restrict__ b_r, int64_t T, int d, int E,
                                                           int k, int mode, int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_w, int32_t* __restrict__ status) {
    extern __shared__ float smem[];
    float* lg = smem;                       // [RT_TOK][E]
    float* part = smem + RT_TOK * E;        // split-K partials (small E only)
    const int64_t t0 = (int64_t)blockIdx.x * RT_TOK;

    if (BF16)
        scores_bf16_mfma<EPL>(static_cast<const uint16_t*>(xv), w_r, t0, T, d, E, lg, part);
    else
        scores_f32(static_cast<const float*>(xv), w_r, t0, T, d, E, lg);
    __syncthreads();

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    for (int r = wave; r < RT_TOK; r += RT_THREADS / 64) {
        const int64_t t = t0 + r;
        if (t >= T) break;
        float v[EPL];
        bool bad = false;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            float g = -INFINITY;
            if (e < E) {
                g = lg[r * E + e] + (b_r ? b_r[e] : 0.f);
                bad |= !isfinite(g);
            }
            v[j] = g;
        }
        bad = __any(bad);
        if (bad) {
            if (lane < k) {
                topk_ids[t * k + lane] = lane;
                topk_w[t * k + lane] = 0.f;
            }
            if (lane == 0) *status = MOE_ERR_NONFINITE_LOGIT;
            continue;
        }
        // k rounds of a wave arg-max over (score key, lower id first).
        uint32_t taken = 0;
        int my_e = 0;
        float my_g = 0.f;
        for (int s = 0; s < k; ++s) {
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
            // recover the score of the winner from its owner lane
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
        float wgt;
        if (mode == MOE_GATE_SWITCH) {
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (lane + 64 * j < E) z += expf(v[j] - g_top);
            z = wave_sum(z);
            wgt = expf(my_g - g_top) / z;
        } else {
            const float ez = lane < k ? expf(my_g - g_top) : 0.f;
            const float z = wave_sum(ez);
            wgt = ez / z;
        }
        if (lane < k) {
            topk_ids[t * k + lane] = my_e;
            topk_w[t * k + lane] = wgt;
        }
    }
}

template <int EPL>
hipError_t launch_route_epl(const moe_dims& s, const void* x, const float* w_r, const float* b_r, int32_t* ids,
                            float* w, int32_t* status, hipStream_t st) {
    const int NT = (s.E + 15) / 16;
    const int CG = NT < 4 ? NT : 4;
    const int KS = 4 / CG;
    size_t lds = sizeof(float) * RT_TOK * s.E;
    if (s.dtype == MOE_BF16 && KS > 1) lds += sizeof(float) * KS * RT_TOK * NT * 16;
    const unsigned grid = (unsigned)((s.T + RT_TOK - 1) / RT_TOK);
    if (s.dtype == MOE_BF16)
        hipLaunchKernelGGL((route_kernel<EPL, true>), dim3(grid), dim3(RT_THREADS), lds, st, x, w_r, b_r, s.T, s.d,
                           s.E, s.k, s.gate_mode, ids, w, status);
    else
        hipLaunchKernelGGL((route_kernel<EPL, false>), dim3(grid), dim3(RT_THREADS), lds, st, x, w_r, b_r, s.T, s.d,
                           s.E, s.k, s.gate_mode, ids, w, status);
    return hipGetLastError();
}

}  // namespace

namespace moe_kernels {

hipError_t launch_route(const moe_dims& s, const void* x, const float* w_r, const float* b_r, int32_t* topk_ids,
                        float* topk_w, int32_t* status, hipStream_t st) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, st, status, 1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.T == 0) return e;
    if (s.E <= 64) return launch_route_epl<1>(s, x, w_r, b_r, topk_ids, topk_w, status, st);
    if (s.E <= 128) return launch_route_epl<2>(s, x, w_r, b_r, topk_ids, topk_w, status, st);
    if (s.E <= 256) return launch_route_epl<4>(s, x, w_r, b_r, topk_ids, topk_w, status, st);
    if (s.E <= 512) return launch_route_epl<8>(s, x, w_r, b_r, topk_ids, topk_w, status, st);
    return launch_route_epl<16>(s, x, w_r, b_r, topk_ids, topk_w, status, st);
}

}  // namespace moe_kernels
