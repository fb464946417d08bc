// Grouped expert GEMMs over ragged per-expert row ranges.
//
//   GEMM1 (gate/up + SwiGLU):  h = SiLU(x_e W_gate,e^T) (*) (x_e W_up,e^T)
//   GEMM2 (down):              H = h_e W_down,e^T
// ("MoE token routing" §3 SwiGLU expert; "LLM from scratch" ch. 36 §36.1 gated
// expert and Algorithm 36.1 expert step: each expert runs only on its accepted
// rows.)  Rows of expert e are [offsets[e], offsets[e+1]); the tile schedule is
// derived on the device from `offsets`, so no host round trip sits between
// dispatch and the GEMMs.
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * 256 threads = 2 x 2 waves; workgroup tile 256 rows x BN output columns,
//     K step 64.  GEMM1 loads BN gate rows and BN up rows of the weights into the
//     same B tile so that each lane owns the gate and the up value of the same
//     output element and applies SiLU(g) * u in registers before one bf16 store.
//   * A and B tiles are staged through LDS (double-buffered, one barrier per K
//     step), 16-byte chunks XOR-swizzled by row so that the 16-byte operand reads
//     of 32 consecutive rows hit distinct banks.
//   * Workgroups are renumbered so that every XCD (workgroup id mod 8) receives
//     a contiguous run of the work list, ordered (n super-tile of 8, m tile,
//     n tile): the workgroups an XCD runs together share A row tiles and expert
//     weight tiles in its own L2.
// fp32 path: a plain LDS-tiled fp32 FMA kernel (64 x 64 tiles, 4 x 4 per thread).
#include "common.h"

namespace {

constexpr int XCDS = 8;
constexpr int NSUPER = 8;

struct TileCoord {
    int g, nt;
    int64_t row_start, row_end;
};

__device__ __forceinline__ bool tile_coords(int b, const int32_t* __restrict__ offsets,
                                            const int32_t* __restrict__ tprefix, int G, int64_t nrows, int BM, int NT,
                                            TileCoord& tc) {
    const int MT = offsets ? tprefix[G] : (int)((nrows + BM - 1) / BM);
    const int total = MT * NT;
    if (b >= total) return false;
    const int x = b % XCDS, j = b / XCDS;
    const int q = total / XCDS, rmd = total % XCDS;
    const int w = x * q + min(x, rmd) + j;
    const int per_super = MT * NSUPER;
    const int ns = w / per_super;
    const int rem = w - ns * per_super;
    const int width = min(NSUPER, NT - ns * NSUPER);
    const int mtg = rem / width;
    tc.nt = ns * NSUPER + rem % width;
    if (offsets) {
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tprefix[mid] <= mtg) lo = mid;
            else hi = mid - 1;
        }
        tc.g = lo;
        tc.row_start = (int64_t)offsets[lo] + (int64_t)(mtg - tprefix[lo]) * BM;
        tc.row_end = offsets[lo + 1];
    } else {
        tc.g = 0;
        tc.row_start = (int64_t)mtg * BM;
        tc.row_end = nrows;
    }
    return true;
}

// tprefix[g] = sum_{g' < g} ceil(rows(g') / BM); one workgroup, G <= 1024.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets, int G, int BM,
                                                           int32_t* __restrict__ tprefix) {
    __shared__ int s_sum[16];
    const int g = threadIdx.x, wave = g / 64, lane = g % 64;
    int cnt = 0;
    if (g < G) {
        const int rows = offsets[g + 1] - offsets[g];
        cnt = rows > 0 ? (rows + BM - 1) / BM : 0;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, MOE_WAVE);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_sum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < 16; ++w) {
        if (w < wave) before += s_sum[w];
        total += s_sum[w];
    }
    if (g < G) tprefix[g] = before + incl - cnt;
    if (g == 0) tprefix[G] = total;
}

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM
// ---------------------------------------------------------------------------

template <int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ B0,
                                                           const uint16_t* __restrict__ B1, void* __restrict__ Cout,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ tprefix, int G, int64_t nrows,
                                                           int N, int K) {
    constexpr int BK = 64, CPR = BK / 8;          // 16-byte chunks per tile row
    constexpr int NOPS = SWIGLU ? 2 : 1;
    constexpr int BROWS = NOPS * BN;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MT = WM / 32, NTW = WN / 32;
    constexpr int A_LD = BM * CPR / 256, B_LD = BROWS * CPR / 256;
    constexpr int ROWS_PER_PASS = 256 / CPR;      // 32 tile rows per load pass
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile shape");

    __shared__ uint4 sA[2][BM * CPR];
    __shared__ uint4 sB[2][BROWS * CPR];

    TileCoord tc;
    const int NT = (N + BN - 1) / BN;
    if (!tile_coords(blockIdx.x, offsets, tprefix, G, nrows, BM, NT, tc)) return;

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = tc.nt * BN;
    const int64_t wstride = (int64_t)N * K;
    const uint16_t* Bg = B0 + (int64_t)tc.g * wstride;
    const uint16_t* Bu = SWIGLU ? B1 + (int64_t)tc.g * wstride : nullptr;

    // Global -> LDS load plan: thread owns chunk column c and rows r0 + 32 i.
    const int c = tid % CPR, r0 = tid / CPR;
    const int swz = (c ^ (r0 % 8));
    const int lds_off = r0 * CPR + swz;
    const uint16_t* a_base = A + (tc.row_start + r0) * (int64_t)K + c * 8;
    uint32_t a_ok = 0, b_ok = 0;
    const uint16_t* b_ptr[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
        if (tc.row_start + r0 + ROWS_PER_PASS * i < tc.row_end) a_ok |= 1u << i;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = r0 + ROWS_PER_PASS * i;
        const int op = (SWIGLU && r >= BN) ? 1 : 0;
        const int n = n0 + r - op * BN;
        if (n < N) b_ok |= 1u << i;
        b_ptr[i] = (op ? Bu : Bg) + (int64_t)(n < N ? n : 0) * K + c * 8;
    }

    uint4 ra[A_LD], rb[B_LD];
    const uint4 zero4 = {0u, 0u, 0u, 0u};
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
        const bool kok = k0 + c * 8 < K;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = (kok && ((a_ok >> i) & 1u))
                        ? *reinterpret_cast<const uint4*>(a_base + (int64_t)ROWS_PER_PASS * i * K + k0)
                        : zero4;
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[i] = (kok && ((b_ok >> i) & 1u)) ? *reinterpret_cast<const uint4*>(b_ptr[i] + k0) : zero4;
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) sA[buf][lds_off + ROWS_PER_PASS * CPR * i] = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) sB[buf][lds_off + ROWS_PER_PASS * CPR * i] = rb[i];
    };

    floatx16_t acc[NOPS][MT][NTW];
#pragma unroll
    for (int o = 0; o < NOPS; ++o)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[o][i][j][v] = 0.f;

    const int KT = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();

    const int lrow = lane % 32, lhalf = lane / 32;
    const int rswz = lrow % 8;
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const uint4* As = sA[buf];
        const uint4* Bs = sB[buf];
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int cc = (2 * s + lhalf) ^ rswz;
            bf16x8_t a[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) a[i] = as_bf16x8(As[(wm * WM + i * 32 + lrow) * CPR + cc]);
#pragma unroll
            for (int o = 0; o < NOPS; ++o) {
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const bf16x8_t b = as_bf16x8(Bs[(o * BN + wn * WN + j * 32 + lrow) * CPR + cc]);
#pragma unroll
                    for (int i = 0; i < MT; ++i)
                        acc[o][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[o][i][j], 0, 0, 0);
                }
            }
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator: lane holds column (lane % 32) and rows
    // 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int col = n0 + wn * WN + j * 32 + lrow;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = tc.row_start + wm * WM + i * 32 + 8 * (v / 4) + 4 * lhalf + (v % 4);
                if (row < tc.row_end && col < N) {
                    if (SWIGLU) {
                        const float hval = silu_f32(acc[0][i][j][v]) * acc[NOPS - 1][i][j][v];
                        static_cast<uint16_t*>(Cout)[row * N + col] = (uint16_t)f32_to_bf16_bits(hval);
                    } else {
                        static_cast<float*>(Cout)[row * N + col] = acc[0][i][j][v];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM (plain FMA)
// ---------------------------------------------------------------------------

template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B0,
                                                       const float* __restrict__ B1, float* __restrict__ Cout,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ tprefix, int G, int64_t nrows,
                                                       int N, int K) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[SWIGLU ? 2 : 1][BK][BN + 4];
    TileCoord tc;
    const int NT = (N + BN - 1) / BN;
    if (!tile_coords(blockIdx.x, offsets, tprefix, G, nrows, BM, NT, tc)) return;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    const int n0 = tc.nt * BN;
    const int64_t wstride = (int64_t)N * K;
    const float* Bg = B0 + (int64_t)tc.g * wstride;
    const float* Bu = SWIGLU ? B1 + (int64_t)tc.g * wstride : nullptr;
    float acc[2][4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        for (int p = tid; p < BM * BK; p += 256) {
            const int r = p / BK, kk = p % BK;
            const int64_t row = tc.row_start + r;
            As[kk][r] = (row < tc.row_end && k0 + kk < K) ? A[row * K + k0 + kk] : 0.f;
            const int n = n0 + r;
            Bs[0][kk][r] = (n < N && k0 + kk < K) ? Bg[(int64_t)n * K + k0 + kk] : 0.f;
            if (SWIGLU) Bs[SWIGLU ? 1 : 0][kk][r] = (n < N && k0 + kk < K) ? Bu[(int64_t)n * K + k0 + kk] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4], u[4];
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
            for (int j = 0; j < 4; ++j) b[j] = Bs[0][kk][tx * 4 + j];
            if (SWIGLU)
                for (int j = 0; j < 4; ++j) u[j] = Bs[SWIGLU ? 1 : 0][kk][tx * 4 + j];
            for (int i = 0; i < 4; ++i)
                for (int j = 0; j < 4; ++j) {
                    acc[0][i][j] = fmaf(a[i], b[j], acc[0][i][j]);
                    if (SWIGLU) acc[1][i][j] = fmaf(a[i], u[j], acc[1][i][j]);
                }
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        const int64_t row = tc.row_start + ty * 4 + i;
        if (row >= tc.row_end) continue;
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + tx * 4 + j;
            if (col >= N) continue;
            Cout[row * N + col] = SWIGLU ? silu_f32(acc[0][i][j]) * acc[1][i][j] : acc[0][i][j];
        }
    }
}

constexpr int BF16_BM = 256;
constexpr int BF16_BN1 = 128;   // GEMM1 output columns per tile (256 weight rows: gate + up)
constexpr int BF16_BN2 = 256;   // GEMM2 output columns per tile
constexpr int F32_BM = 64, F32_BN = 64;

hipError_t prep_tiles(const int32_t* offsets, int G, int BM, void* ws, hipStream_t st) {
    if (!offsets) return hipSuccess;
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, G, BM, static_cast<int32_t*>(ws));
    return hipGetLastError();
}

unsigned grid_size(const int32_t* offsets, int G, int64_t max_rows, int BM, int N, int BN) {
    const int64_t mt = (max_rows + BM - 1) / BM + (offsets ? G : 0);
    const int64_t nt = (N + BN - 1) / BN;
    return (unsigned)(mt * nt);
}

}  // namespace

namespace moe_kernels {

size_t gemm_ws_bytes(int G) { return (((size_t)(G + 1) * sizeof(int32_t)) + 255) & ~(size_t)255; }

hipError_t launch_gemm1(int dtype, const void* A, const int32_t* offsets, int G, int64_t max_rows, const void* w_gate,
                        const void* w_up, void* h, int N, int K, void* ws, hipStream_t st) {
    const int BM = dtype == MOE_BF16 ? BF16_BM : F32_BM;
    const int BN = dtype == MOE_BF16 ? BF16_BN1 : F32_BN;
    hipError_t e = prep_tiles(offsets, G, BM, ws, st);
    if (e != hipSuccess) return e;
    const unsigned grid = grid_size(offsets, G, max_rows, BM, N, BN);
    if (grid == 0) return hipSuccess;
    const int32_t* tp = static_cast<const int32_t*>(ws);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL((gemm_bf16_kernel<BF16_BM, BF16_BN1, true>), dim3(grid), dim3(256), 0, st,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(w_gate),
                           static_cast<const uint16_t*>(w_up), h, offsets, tp, G, max_rows, N, K);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<true>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(A),
                           static_cast<const float*>(w_gate), static_cast<const float*>(w_up),
                           static_cast<float*>(h), offsets, tp, G, max_rows, N, K);
    return hipGetLastError();
}

hipError_t launch_gemm2(int dtype, const void* h, const int32_t* offsets, int G, int64_t max_rows,
                        const void* w_down, float* H, int N, int K, void* ws, hipStream_t st) {
    const int BM = dtype == MOE_BF16 ? BF16_BM : F32_BM;
    const int BN = dtype == MOE_BF16 ? BF16_BN2 : F32_BN;
    hipError_t e = prep_tiles(offsets, G, BM, ws, st);
    if (e != hipSuccess) return e;
    const unsigned grid = grid_size(offsets, G, max_rows, BM, N, BN);
    if (grid == 0) return hipSuccess;
    const int32_t* tp = static_cast<const int32_t*>(ws);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL((gemm_bf16_kernel<BF16_BM, BF16_BN2, false>), dim3(grid), dim3(256), 0, st,
                           static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), nullptr, H,
                           offsets, tp, G, max_rows, N, K);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<false>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(h),
                           static_cast<const float*>(w_down), nullptr, H, offsets, tp, G, max_rows, N, K);
    return hipGetLastError();
}

}  // namespace moe_kernels
