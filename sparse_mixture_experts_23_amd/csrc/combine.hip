// Weighted combine back into token order.
//
//   y[t] = s[t] + sum_{r : row_of[t,r] >= 0} a[t,r] * H[row_of[t,r]]
//
// ("LLM from scratch" ch. 36 Algorithm 36.1 combine step: every accepted record
// is added once, rejected records add nothing and the other weights are not
// renormalised; "MoE token routing" §3 weighted sum; shared expert added
// unweighted, ch. 36 §36.6.)  The scatter-add of the definition is computed as a
// token-major gather: each token's row is written by exactly one wave, summing
// its paths in rank order with fp32 fused multiply-adds, so the result is
// deterministic without atomics.  Overflow variant (ch. 36 §36.4 worked
// example): with renorm_survivors each accepted weight is first divided by the
// sum of the token's accepted weights.  With rerouting a token has 2k records
// (its selection, then its next choices), summed the same way.
#include "common.h"

namespace {

constexpr int COMBINE_U = 4;   // 64-lane column blocks per wave (float4 each; scalar path: floats)
constexpr int COMBINE_PR = 4;  // paths whose rows are loaded together (vector path)

// H1 (nullable): np further K-split partials of H, block p at H1 + p ps; the row
// used is ((H + P_0) + P_1) + ... (the value a caller that folded them into H in
// that order would read).
template <bool VEC4>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ H, const float* __restrict__ H1,
                                                      int np, int64_t ps, const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ w, const float* __restrict__ shared_out,
                                                      float* __restrict__ y, int64_t T, int d, int k,
                                                      int nchunk, int renorm) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;   // (token, column chunk) of this wave
    const int64_t t = gw / nchunk;
    const int chunk = (int)(gw % nchunk);
    if (t >= T) return;
    const int myrow = lane < k ? row_of[t * k + lane] : -1;
    float myw = lane < k ? w[t * k + lane] : 0.f;
    if (renorm) {   // overflow variant: weights over the accepted paths, summed in rank order
        float tot = 0.f;
        for (int r = 0; r < k; ++r)
            if (lane_value(myrow, r) >= 0) tot += lane_value(myw, r);
        if (tot > 0.f) myw = myw / tot;
    }
    if (VEC4) {
        // A wave owns U column blocks of 64 float4: a path's U loads (and its
        // partials') are in flight together; per element the sum is still
        // s + a0 h0 + a1 h1 + ...
        constexpr int U = COMBINE_U;
        const int nv = d / 4;
        const float4* H4 = reinterpret_cast<const float4*>(H);
        const float4* H14 = reinterpret_cast<const float4*>(H1);
        const float4* S4 = reinterpret_cast<const float4*>(shared_out);
        float4* Y4 = reinterpret_cast<float4*>(y);
        // uniform trip count: every lane stays active around lane_value
        for (int c0 = chunk * 64 * U; c0 < (chunk + 1) * 64 * U; c0 += 64 * U) {
            float4 acc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * 64 + lane;
                acc[u] = (shared_out && c < nv) ? S4[t * nv + c] : float4{0.f, 0.f, 0.f, 0.f};
            }
            // COMBINE_PR paths per round: their rows' loads are issued together, then
            // they are added in rank order (a rejected path loads nothing, adds nothing)
            for (int r0 = 0; r0 < k; r0 += COMBINE_PR) {
                int row[COMBINE_PR];
                float a[COMBINE_PR];
                float4 h[COMBINE_PR][U];
#pragma unroll
                for (int q = 0; q < COMBINE_PR; ++q) {
                    row[q] = r0 + q < k ? lane_value(myrow, r0 + q) : -1;
                    a[q] = r0 + q < k ? lane_value(myw, r0 + q) : 0.f;
                    if (row[q] < 0) continue;   // uniform across the wave
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + u * 64 + lane;
                        h[q][u] = c < nv ? H4[(int64_t)row[q] * nv + c] : float4{0.f, 0.f, 0.f, 0.f};
                    }
                    // the first partial's loads are issued with H's (no loop in between)
                    if (np > 0) {
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int c = c0 + u * 64 + lane;
                            const float4 h1 = c < nv ? H14[(int64_t)row[q] * nv + c] : float4{0.f, 0.f, 0.f, 0.f};
                            h[q][u].x += h1.x;
                            h[q][u].y += h1.y;
                            h[q][u].z += h1.z;
                            h[q][u].w += h1.w;
                        }
                    }
                    for (int p = 1; p < np; ++p) {
                        const float4* P4 = H14 + p * (ps / 4);
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int c = c0 + u * 64 + lane;
                            const float4 h1 = c < nv ? P4[(int64_t)row[q] * nv + c] : float4{0.f, 0.f, 0.f, 0.f};
                            h[q][u].x += h1.x;
                            h[q][u].y += h1.y;
                            h[q][u].z += h1.z;
                            h[q][u].w += h1.w;
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < COMBINE_PR; ++q) {
                    if (row[q] < 0) continue;
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        acc[u].x = fmaf(a[q], h[q][u].x, acc[u].x);
                        acc[u].y = fmaf(a[q], h[q][u].y, acc[u].y);
                        acc[u].z = fmaf(a[q], h[q][u].z, acc[u].z);
                        acc[u].w = fmaf(a[q], h[q][u].w, acc[u].w);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * 64 + lane;
                if (c < nv) Y4[t * nv + c] = acc[u];
            }
        }
    } else {
        for (int c0 = chunk * 64 * COMBINE_U; c0 < min(d, (chunk + 1) * 64 * COMBINE_U); c0 += 64) {
            const int c = c0 + lane;
            const bool ok = c < d;
            float acc = (shared_out && ok) ? shared_out[t * d + c] : 0.f;
            for (int r = 0; r < k; ++r) {
                const int row = lane_value(myrow, r);
                const float a = lane_value(myw, r);
                if (row >= 0 && ok) {
                    float h = H[(int64_t)row * d + c];
                    for (int p = 0; p < np; ++p) h += H1[p * ps + (int64_t)row * d + c];
                    acc = fmaf(a, h, acc);
                }
            }
            if (ok) y[t * d + c] = acc;
        }
    }
}

}  // namespace

namespace moe_kernels {

hipError_t launch_combine(const moe_dims& s, const float* H, const float* H1, int np, int64_t part_stride,
                          const int32_t* row_of, const float* topk_w, const float* shared_out, float* y,
                          hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    if (!H1) np = 0;
    // one wave per (token, chunk of COMBINE_U 64-lane column blocks)
    const bool vec4 = s.d % 4 == 0;
    const int cols = vec4 ? s.d / 4 : s.d;
    const int nchunk = (cols + 64 * COMBINE_U - 1) / (64 * COMBINE_U);
    const unsigned grid = (unsigned)((s.T * nchunk + 3) / 4);
    if (vec4)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, st, H, H1, np, part_stride, row_of, topk_w,
                           shared_out, y, s.T, s.d, moe_paths(s), nchunk, s.renorm_survivors);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, st, H, H1, np, part_stride, row_of,
                           topk_w, shared_out, y, s.T, s.d, moe_paths(s), nchunk, s.renorm_survivors);
    return hipGetLastError();
}

}  // namespace moe_kernels
