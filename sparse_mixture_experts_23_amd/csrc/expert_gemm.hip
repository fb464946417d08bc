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
//   * workgroup tile 256 rows x BN output columns.  GEMM1 puts BN gate rows and
//     BN up rows of the weights into one B tile so that each lane owns the gate
//     and the up value of the same output element and applies SiLU(g) * u in
//     registers before a single bf16 store.
//   * main kernel (K % 32 == 0): 8 waves (2 per SIMD), K tiles of 64 (or 32)
//     streamed into an LDS ring by gfx950's direct global->LDS loads; see
//     gemm_bf16_ring_kernel.
//   * fallback kernel (any K % 8 == 0): 4 waves, register-staged loads, K tiles
//     of 64 double-buffered in LDS, zero-filled K tail.
//   * LDS rows are stored with their 16-byte chunks XOR-swizzled by row, so the
//     16-byte operand reads of 32 consecutive rows hit distinct banks.
//   * Workgroups are renumbered so that every XCD (workgroup id mod 8) receives
//     a contiguous run of the work list, ordered (n super-tile of 8, m tile,
//     n tile): the workgroups an XCD runs together share A row tiles and expert
//     weight tiles in its own L2.
// fp32 path: a plain LDS-tiled fp32 FMA kernel (64 x 64 tiles, 4 x 4 per thread).
#include <type_traits>

#include "common.h"

namespace {

constexpr int XCDS = 8;
constexpr int NSUPER = 4;

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
    constexpr int nsup = NSUPER;
    const int per_super = MT * nsup;
    const int ns = w / per_super;
    const int rem = w - ns * per_super;
    const int width = min(nsup, NT - ns * nsup);
    const int mtg = rem / width;
    tc.nt = ns * nsup + rem % width;
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

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef const u32x4_t __attribute__((address_space(1)))* gmem_u32x4;

// 16-byte load through a global-address-space pointer (global_load_dwordx4).
__device__ __forceinline__ uint4 gload16(const uint16_t* p) {
    return __builtin_bit_cast(uint4, *(gmem_u32x4)(p));
}

// LDS chunk swizzle: 16-byte chunk c of tile row r is stored at c ^ swz(r).
// A 32x32x16 operand read has 32 lanes on 32 consecutive rows at one chunk; with
// swz(r) = (r & 7) ^ ((r >> 3) & 1) any 8 consecutive rows hit 8 different
// 16-byte bank groups of a 128-byte window and any 16 consecutive rows hit 16
// different groups of a 256-byte window.
__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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
    const uint16_t* Bu = SWIGLU ? B1 + (int64_t)tc.g * wstride : Bg;

    // Global -> LDS plan: thread owns chunk column c of tile rows r0 + 32 i
    // (ROWS_PER_PASS is a multiple of 16, so every owned row has the same swizzle).
    const int c = tid % CPR, r0 = tid / CPR;
    const int lds_off = r0 * CPR + (c ^ lds_swz(r0));
    const uint16_t* a_src = A + (tc.row_start + r0) * (int64_t)K + c * 8;
    uint32_t a_ok = 0, b_ok = 0;
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
        if (tc.row_start + r0 + ROWS_PER_PASS * i < tc.row_end) a_ok |= 1u << i;
    // B rows: pass i covers tile rows r0 + 32 i; the first BN rows come from B0
    // (gate or down), the next BN from B1 (up).
    constexpr int B_PASS_OP = BN / ROWS_PER_PASS;   // passes per operand
    const uint16_t* b_src0 = Bg + (int64_t)(n0 + r0) * K + c * 8;
    const uint16_t* b_src1 = Bu + (int64_t)(n0 + r0) * K + c * 8;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int n = n0 + r0 + ROWS_PER_PASS * (i % B_PASS_OP);
        if (n < N) b_ok |= 1u << i;
    }

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
    const uint4 zero4 = {0u, 0u, 0u, 0u};
    uint4 ra[A_LD], rb[B_LD];

    // prologue: tile 0
    {
        const bool kok = c * 8 < K;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = (kok && ((a_ok >> i) & 1u)) ? gload16(a_src + (int64_t)ROWS_PER_PASS * i * K) : zero4;
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const uint16_t* src = (i < B_PASS_OP ? b_src0 : b_src1) + (int64_t)ROWS_PER_PASS * (i % B_PASS_OP) * K;
            rb[i] = (kok && ((b_ok >> i) & 1u)) ? gload16(src) : zero4;
        }
#pragma unroll
        for (int i = 0; i < A_LD; ++i) sA[0][lds_off + ROWS_PER_PASS * CPR * i] = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) sB[0][lds_off + ROWS_PER_PASS * CPR * i] = rb[i];
    }
    __syncthreads();

    const int lrow = lane % 32, lhalf = lane / 32;
    const int rswz = lds_swz(lrow);       // tile rows read by this lane are lrow + 32 j
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            const int k0 = (kt + 1) * BK;
            const bool kok = k0 + c * 8 < K;
#pragma unroll
            for (int i = 0; i < A_LD; ++i)
                ra[i] = (kok && ((a_ok >> i) & 1u)) ? gload16(a_src + (int64_t)ROWS_PER_PASS * i * K + k0) : zero4;
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                const uint16_t* src =
                    (i < B_PASS_OP ? b_src0 : b_src1) + (int64_t)ROWS_PER_PASS * (i % B_PASS_OP) * K + k0;
                rb[i] = (kok && ((b_ok >> i) & 1u)) ? gload16(src) : zero4;
            }
        }
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
        if (more) {
#pragma unroll
            for (int i = 0; i < A_LD; ++i) sA[buf ^ 1][lds_off + ROWS_PER_PASS * CPR * i] = ra[i];
#pragma unroll
            for (int i = 0; i < B_LD; ++i) sB[buf ^ 1][lds_off + ROWS_PER_PASS * CPR * i] = rb[i];
        }
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
// helpers of the pipelined bf16 kernel
// ---------------------------------------------------------------------------

// Swizzle of the 4 chunks of a 64-byte tile row: any 8 consecutive rows read at
// one chunk hit 8 different 16-byte bank groups of a 128-byte window, and any 16
// consecutive rows 16 different groups of a 256-byte window.
__device__ __forceinline__ int lds_swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// The same global->LDS load issued from a tiny asm statement.  It has no
// register outputs (the data goes to LDS), so it does not touch the rule that
// asm loads must wait for their outputs; what it changes is that the compiler
// no longer sees an LDS write it cannot place, and so it stops making every LDS
// read wait for all of these loads.  Callers order them with explicit vmcnt
// waits and barriers.  M0 (the LDS base of the load) is saved and restored.
__device__ __forceinline__ void dma16_async(const uint16_t* src, uint32_t lds_wave_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_wave_addr)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM: 8 waves, global->LDS ring, barrier per K tile
// ---------------------------------------------------------------------------
//
// Workgroup tile 256 rows x BN output columns (GEMM1: 128 gate + 128 up weight
// rows in one B tile), 8 waves = 2 per SIMD, each owning a 64 x 128 tile of
// 32x32x16 MFMA accumulators.  K tiles (BK = 64: 2 LDS stages; BK = 32: 4
// stages; 128 KB either way) are written straight into LDS by dma16_async, one
// full 128-byte line per row segment at BK = 64.  The compiler schedules the
// ordinary LDS operand reads of the next K substep between the MFMAs of the
// current one.  The barrier sits before the last substep of a tile: by then
// every wave has read all of tile kt, so its stage is refilled with tile
// kt + STAGES at once, and the next tile's first operands are read while the
// last substep multiplies.
// Wait until at most n K tiles of LOADS global->LDS loads each are still in flight.
template <int LOADS>
__device__ __forceinline__ void wait_tiles(int n) {
    if (n >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(3 * LOADS) : "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(2 * LOADS) : "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"i"(LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Barrier after this wave's LDS reads have completed (no wave still reads a
// stage when the next load into it is issued).
__device__ __forceinline__ void lds_barrier_reads_done() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int BM, int BN, bool SWIGLU, int WGM, int WGN, int BK>
__global__ __launch_bounds__(WGM * WGN * 64, 1) void gemm_bf16_ring_kernel(const uint16_t* __restrict__ A,
                                                                         const uint16_t* __restrict__ B0,
                                                                         const uint16_t* __restrict__ B1,
                                                                         void* __restrict__ Cout,
                                                                         const int32_t* __restrict__ offsets,
                                                                         const int32_t* __restrict__ tprefix, int G,
                                                                         int64_t nrows, int N, int K) {
    constexpr int NTHR = WGM * WGN * 64;
    constexpr int CPR = BK / 8;                     // 16-byte chunks per tile row (4 or 8)
    constexpr int RPI = 64 / CPR;                   // tile rows per wave load instruction
    constexpr int STAGES = BK == 32 ? 4 : 2;        // 128 KB of LDS either way
    constexpr int SUB = BK / 16;                    // MFMA K substeps per tile
    constexpr int NOPS = SWIGLU ? 2 : 1;
    constexpr int BROWS = NOPS * BN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int MT = WM / 32, NTW = WN / 32;
    constexpr int A_CH = BM * CPR, B_CH = BROWS * CPR;
    constexpr int A_LD = A_CH / NTHR, B_LD = B_CH / NTHR;    // DMA per thread per tile
    constexpr int LOADS = A_LD + B_LD;
    constexpr int WAVES = WGM * WGN;
    static_assert(BK == 32 || BK == 64, "K tile");
    static_assert(A_CH % NTHR == 0 && B_CH % NTHR == 0 && 3 * LOADS <= 63, "load plan");

    __shared__ uint4 sA[STAGES * A_CH];
    __shared__ uint4 sB[STAGES * B_CH];

    TileCoord tc;
    const int NT = (N + BN - 1) / BN;
    if (!tile_coords(blockIdx.x, offsets, tprefix, G, nrows, BM, NT, tc)) return;

    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int wm = wave / WGN, wn = wave % WGN;
    const int n0 = tc.nt * BN;
    const int64_t wstride = (int64_t)N * K;
    const uint16_t* Bg = B0 + (int64_t)tc.g * wstride;
    const uint16_t* Bu = SWIGLU ? B1 + (int64_t)tc.g * wstride : Bg;

    auto swz = [](int r) { return CPR == 4 ? lds_swz4(r) : lds_swz(r); };
    // DMA plan: instruction i of wave w fills chunks [(WAVES i + w) * 64, +64) =
    // RPI tile rows; this lane fills row (WAVES i + w) * RPI + lane / CPR at
    // physical chunk lane % CPR, i.e. logical chunk (lane % CPR) ^ swz(row).
    const uint16_t* a_src[A_LD];
    const uint16_t* b_src[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int row = (WAVES * i + wave) * RPI + lane / CPR;
        int64_t gr = tc.row_start + row;
        if (gr >= tc.row_end) gr = tc.row_start;
        a_src[i] = A + gr * K + ((lane % CPR) ^ swz(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int row = (WAVES * i + wave) * RPI + lane / CPR;
        const int op = row / BN;
        int n = n0 + row % BN;
        if (n >= N) n = n0;
        b_src[i] = (op ? Bu : Bg) + (int64_t)n * K + ((lane % CPR) ^ swz(row)) * 8;
    }
    const uint32_t sA_addr = lds_byte_addr(sA), sB_addr = lds_byte_addr(sB);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto issue = [&](int kt, int stage) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            dma16_async(a_src[i] + k0, sA_addr + (uint32_t)((stage * A_CH + (WAVES * i + wave_u) * 64) * 16));
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            dma16_async(b_src[i] + k0, sB_addr + (uint32_t)((stage * B_CH + (WAVES * i + wave_u) * 64) * 16));
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

    const int KT = K / BK;
    for (int t = 0; t < STAGES && t < KT; ++t) issue(t, t);

    const int lrow = lane % 32, lhalf = lane / 32;
    const int rswz = swz(lrow);    // operand rows are lrow + multiples of 32
    auto read_ops = [&](int stage, int s, bf16x8_t (&a)[MT], bf16x8_t (&b)[NOPS][NTW]) {
        const uint4* As = sA + stage * A_CH;
        const uint4* Bs = sB + stage * B_CH;
        const int cc = (2 * s + lhalf) ^ rswz;
#pragma unroll
        for (int i = 0; i < MT; ++i) a[i] = as_bf16x8(As[(wm * WM + i * 32 + lrow) * CPR + cc]);
#pragma unroll
        for (int o = 0; o < NOPS; ++o)
#pragma unroll
            for (int j = 0; j < NTW; ++j) b[o][j] = as_bf16x8(Bs[(o * BN + wn * WN + j * 32 + lrow) * CPR + cc]);
    };
    auto mma = [&](const bf16x8_t (&a)[MT], const bf16x8_t (&b)[NOPS][NTW]) {
#pragma unroll
        for (int o = 0; o < NOPS; ++o)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[o][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[o][j], acc[o][i][j], 0, 0, 0);
    };

    wait_tiles<LOADS>(min(STAGES - 1, KT - 1));
    lds_barrier_reads_done();
    bf16x8_t xa[MT], xb[NOPS][NTW], ya[MT], yb[NOPS][NTW];
    read_ops(0, 0, xa, xb);
    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt % STAGES;
        // substeps 0 .. SUB-2: multiply x while reading the next substep into y, then swap
#pragma unroll
        for (int s = 0; s + 1 < SUB; ++s) {
            if (s % 2 == 0) {
                read_ops(stage, s + 1, ya, yb);
                mma(xa, xb);
            } else {
                read_ops(stage, s + 1, xa, xb);
                mma(ya, yb);
            }
        }
        // last substep: every wave has now read all of tile kt -> barrier, refill its
        // stage, and read the next tile's first substep while multiplying
        auto& la = (SUB % 2 == 0) ? ya : xa;
        auto& lb = (SUB % 2 == 0) ? yb : xb;
        auto& na = (SUB % 2 == 0) ? xa : ya;
        auto& nb = (SUB % 2 == 0) ? xb : yb;
        if (kt + 1 < KT) {
            wait_tiles<LOADS>(min(STAGES - 2, KT - 2 - kt));
            lds_barrier_reads_done();
            if (kt + STAGES < KT) issue(kt + STAGES, stage);
            read_ops((kt + 1) % STAGES, 0, na, nb);
        }
        mma(la, lb);
        if (SUB % 2 == 1) {   // keep "x = operands of substep 0" for the next tile
#pragma unroll
            for (int i = 0; i < MT; ++i) xa[i] = ya[i];
#pragma unroll
            for (int o = 0; o < NOPS; ++o)
#pragma unroll
                for (int j = 0; j < NTW; ++j) xb[o][j] = yb[o][j];
        }
    }

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

template <int BM, int BN, bool SWIGLU>
void launch_ring(unsigned grid, hipStream_t st, const uint16_t* A, const uint16_t* B0, const uint16_t* B1, void* C,
                 const int32_t* offsets, const int32_t* tp, int G, int64_t nrows, int N, int K) {
    if (K % 64 == 0)
        hipLaunchKernelGGL((gemm_bf16_ring_kernel<BM, BN, SWIGLU, 4, 2, 64>), dim3(grid), dim3(512), 0, st, A, B0, B1,
                           C, offsets, tp, G, nrows, N, K);
    else
        hipLaunchKernelGGL((gemm_bf16_ring_kernel<BM, BN, SWIGLU, 4, 2, 32>), dim3(grid), dim3(512), 0, st, A, B0, B1,
                           C, offsets, tp, G, nrows, N, K);
}

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
    if (dtype == MOE_BF16 && K % 32 == 0)
        launch_ring<BF16_BM, BF16_BN1, true>(grid, st,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(w_gate),
                           static_cast<const uint16_t*>(w_up), h, offsets, tp, G, max_rows, N, K);
    else if (dtype == MOE_BF16)
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
    if (dtype == MOE_BF16 && K % 32 == 0)
        launch_ring<BF16_BM, BF16_BN2, false>(grid, st,
                           static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), nullptr, H,
                           offsets, tp, G, max_rows, N, K);
    else if (dtype == MOE_BF16)
        hipLaunchKernelGGL((gemm_bf16_kernel<BF16_BM, BF16_BN2, false>), dim3(grid), dim3(256), 0, st,
                           static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), nullptr, H,
                           offsets, tp, G, max_rows, N, K);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<false>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(h),
                           static_cast<const float*>(w_down), nullptr, H, offsets, tp, G, max_rows, N, K);
    return hipGetLastError();
}

}  // namespace moe_kernels
