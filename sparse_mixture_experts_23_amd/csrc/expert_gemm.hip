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
//   * main kernel (K % 32 == 0): 8 waves (2 per SIMD), K tiles of 32 streamed
//     into a 4-stage LDS ring by gfx950's direct global->LDS loads, so three
//     tiles are in flight while one is multiplied; see gemm_bf16_pipe_kernel.
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

__device__ __forceinline__ void dma16(const uint16_t* src, uint4* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                     (void __attribute__((address_space(3)))*)lds_wave_base, 16, 0, 0);
}

// Workgroup barrier without the memory fence __syncthreads() adds: the fence
// would make the compiler wait for every outstanding global->LDS load.  Callers
// wait for the loads they need with an explicit vmcnt first; the empty asm
// statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM: 8 waves, 4-stage global->LDS pipeline
// ---------------------------------------------------------------------------
//
// Fast path for K % 32 == 0.  Three K tiles stream into LDS by
// global_load_lds_dwordx4 while a fourth is multiplied, so memory latency is
// covered by three tiles of work and costs no staging registers.  The compiler
// cannot tell which LDS stage a global->LDS load writes and would make every
// LDS read wait for all loads in flight; the operand reads are therefore issued
// from small asm blocks (each ends with its own lgkmcnt wait, so its outputs
// are complete when it returns), and the loads are waited for explicitly with
// vmcnt before the stage barrier.  With 2 waves per SIMD each wave keeps a
// 64 x 128 accumulator tile, and the two waves cover each other's LDS waits.

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Six 16-byte LDS reads (2 A operands from one base, 4 B operands from another)
// at immediate byte offsets; returns after all six have landed.
template <int A0, int A1, int B0, int B1, int B2, int B3>
__device__ __forceinline__ void lds_read6(uint32_t a_addr, uint32_t b_addr, u32x4_t& a0, u32x4_t& a1, u32x4_t& b0,
                                          u32x4_t& b1, u32x4_t& b2, u32x4_t& b3) {
    asm volatile(
        "ds_read_b128 %0, %6 offset:%8\n\t"
        "ds_read_b128 %1, %6 offset:%9\n\t"
        "ds_read_b128 %2, %7 offset:%10\n\t"
        "ds_read_b128 %3, %7 offset:%11\n\t"
        "ds_read_b128 %4, %7 offset:%12\n\t"
        "ds_read_b128 %5, %7 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
        : "v"(a_addr), "v"(b_addr), "i"(A0), "i"(A1), "i"(B0), "i"(B1), "i"(B2), "i"(B3)
        : "memory");
}

template <int N_OUTSTANDING_LOADS>
__device__ __forceinline__ void wait_vmcnt_n() {
    if constexpr (N_OUTSTANDING_LOADS == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N_OUTSTANDING_LOADS == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N_OUTSTANDING_LOADS == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else static_assert(N_OUTSTANDING_LOADS == 0, "unsupported wait count");
}

template <int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(512, 1) void gemm_bf16_pipe_kernel(const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ B0,
                                                                const uint16_t* __restrict__ B1,
                                                                void* __restrict__ Cout,
                                                                const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ tprefix, int G,
                                                                int64_t nrows, int N, int K) {
    constexpr int WGM = 4, WGN = 2;                   // 8 waves
    constexpr int BK = 32, CPR = BK / 8, ROWB = BK * 2;   // 64-byte tile rows
    constexpr int STAGES = 4;
    constexpr int NOPS = SWIGLU ? 2 : 1;
    constexpr int BROWS = NOPS * BN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int MT = WM / 32, NTW = WN / 32;
    static_assert(MT == 2 && NOPS * NTW == 4, "operand reads are laid out for 2 A and 4 B operands");
    constexpr int A_CH = BM * CPR, B_CH = BROWS * CPR;          // chunks per stage
    constexpr int A_LD = A_CH / 512, B_LD = B_CH / 512;          // DMA per thread per tile
    static_assert(A_LD + B_LD == 4, "wait counts assume 4 loads per thread per tile");
    constexpr int A_STAGE_BYTES = A_CH * 16, B_STAGE_BYTES = B_CH * 16;

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

    // DMA plan: instruction i of wave w fills chunks [(8 i + w) * 64, +64) = 16 tile
    // rows; this lane fills row (8 i + w) * 16 + lane / 4 at physical chunk
    // lane % 4, i.e. logical chunk (lane % 4) ^ swz(row).
    const int lrow16 = lane / 4;
    const int lchunk = (lane % 4) ^ lds_swz4(lrow16);
    const uint16_t* a_src[A_LD];
    const uint16_t* b_src[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int row = (8 * i + wave) * 16 + lrow16;
        int64_t gr = tc.row_start + row;
        if (gr >= tc.row_end) gr = tc.row_start;
        a_src[i] = A + gr * K + lchunk * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int row = (8 * i + wave) * 16 + lrow16;
        const int op = row / BN;
        int n = n0 + row % BN;
        if (n >= N) n = n0;
        b_src[i] = (op ? Bu : Bg) + (int64_t)n * K + lchunk * 8;
    }
    auto issue = [&](int kt, int stage) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) dma16(a_src[i] + k0, sA + stage * A_CH + (8 * i + wave) * 64);
#pragma unroll
        for (int i = 0; i < B_LD; ++i) dma16(b_src[i] + k0, sB + stage * B_CH + (8 * i + wave) * 64);
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
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
        if (t < KT) issue(t, t);

    // Operand read addresses (stage 0, substep 0).  Substep 1 reads chunk cc ^ 2.
    const int lrow = lane % 32, lhalf = lane / 32;
    const int cc0 = lhalf ^ lds_swz4(lrow);
    const uint32_t a_base = lds_byte_addr(sA) + (wm * WM + lrow) * ROWB;
    const uint32_t b_base = lds_byte_addr(sB) + (wn * WN + lrow) * ROWB;
    const uint32_t a_s[2] = {a_base + cc0 * 16, a_base + (cc0 ^ 2) * 16};
    const uint32_t b_s[2] = {b_base + cc0 * 16, b_base + (cc0 ^ 2) * 16};
    // B operand (o, j) sits (o * BN + j * 32) rows further; A operand i, i * 32 rows.
    constexpr int BO1 = (NOPS == 2 ? 0 * BN + 1 * 32 : 1 * 32) * ROWB;
    constexpr int BO2 = (NOPS == 2 ? 1 * BN + 0 * 32 : 2 * 32) * ROWB;
    constexpr int BO3 = (NOPS == 2 ? 1 * BN + 1 * 32 : 3 * 32) * ROWB;

    auto mma = [&](const u32x4_t& a0, const u32x4_t& a1, const u32x4_t& b0, const u32x4_t& b1, const u32x4_t& b2,
                   const u32x4_t& b3) {
        const bf16x8_t av[2] = {__builtin_bit_cast(bf16x8_t, a0), __builtin_bit_cast(bf16x8_t, a1)};
        const bf16x8_t bv[4] = {__builtin_bit_cast(bf16x8_t, b0), __builtin_bit_cast(bf16x8_t, b1),
                                __builtin_bit_cast(bf16x8_t, b2), __builtin_bit_cast(bf16x8_t, b3)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int o = q / NTW, j = q % NTW;
#pragma unroll
            for (int i = 0; i < MT; ++i)
                acc[o][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[q], acc[o][i][j], 0, 0, 0);
        }
    };

    auto step = [&](auto stage_c, int kt) {
        constexpr int S = decltype(stage_c)::value;
        const int later = min(STAGES - 2, KT - 1 - kt);
        if (later >= 2) wait_vmcnt_n<8>();
        else if (later == 1) wait_vmcnt_n<4>();
        else wait_vmcnt_n<0>();
        lds_barrier();
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (S + STAGES - 1) % STAGES);
        constexpr int AO = S * A_STAGE_BYTES, BOF = S * B_STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            u32x4_t a0, a1, b0, b1, b2, b3;
            lds_read6<AO, AO + 32 * ROWB, BOF, BOF + BO1, BOF + BO2, BOF + BO3>(a_s[s], b_s[s], a0, a1, b0, b1, b2,
                                                                               b3);
            mma(a0, a1, b0, b1, b2, b3);
        }
    };
    for (int kt = 0; kt < KT; kt += STAGES) {
        step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < KT) step(std::integral_constant<int, 1>{}, kt + 1);
        if (kt + 2 < KT) step(std::integral_constant<int, 2>{}, kt + 2);
        if (kt + 3 < KT) step(std::integral_constant<int, 3>{}, kt + 3);
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
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BF16_BM, BF16_BN1, true>), dim3(grid), dim3(512), 0, st,
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
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BF16_BM, BF16_BN2, false>), dim3(grid), dim3(512), 0, st,
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
