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
//   * main kernel (K % 64 == 0): 8 waves (2 per SIMD), K tiles of 64 streamed
//     into LDS by gfx950's direct global->LDS loads (two activation stages,
//     three weight stages, so the weights stream two K tiles ahead), the
//     steady-state K tile written as one scheduled asm block; see
//     gemm_bf16_asm_kernel.
//   * fallback kernel (any K % 8 == 0): 4 waves, register-staged loads, K tiles
//     of 64 double-buffered in LDS, zero-filled K tail.
//   * LDS rows are stored with their 16-byte chunks XOR-swizzled by row, so the
//     16-byte operand reads of 32 consecutive rows hit distinct banks.
//   * Workgroups are renumbered so that every XCD (workgroup id mod 8) receives
//     a contiguous run of the work list, ordered (n super-tile, m tile, n tile):
//     the workgroups an XCD runs together share A row tiles and expert weight
//     tiles in its own L2.  The super-tile is 4 column tiles wide, 16 for GEMM2
//     when the groups average at most one row tile.
// fp32 path: a plain LDS-tiled fp32 FMA kernel (64 x 64 tiles, 4 x 4 per thread).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace {

constexpr int XCDS = 8;
// CUs the GEMM2 K-split rule plans for (MI355X; a fixed figure, so that workspace
// sizes depend on the shape alone)
constexpr int MOE_GEMM_CUS = 256;
constexpr int NSUPER = 4;

struct TileCoord {
    int g, nt;
    int64_t row_start, row_end;
};

// Work item w of the list (n super-tile, m tile, n tile) -> tile.
__device__ __forceinline__ void tile_of_item(int w, const int32_t* __restrict__ offsets,
                                             const int32_t* __restrict__ tprefix, int G, int64_t nrows, int BM,
                                             int NT, int MT, TileCoord& tc, int nsup) {
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
}

__device__ __forceinline__ int tile_count(const int32_t* __restrict__ offsets, const int32_t* __restrict__ tprefix,
                                          int G, int64_t nrows, int BM) {
    return offsets ? tprefix[G] : (int)((nrows + BM - 1) / BM);
}

// Static schedule: workgroup b takes item w of XCD x = b % 8's contiguous run.
__device__ __forceinline__ bool tile_coords(int b, const int32_t* __restrict__ offsets,
                                            const int32_t* __restrict__ tprefix, int G, int64_t nrows, int BM, int NT,
                                            TileCoord& tc, int nsup = NSUPER) {
    const int MT = tile_count(offsets, tprefix, G, nrows, BM);
    const int total = MT * NT;
    if (b >= total) return false;
    const int x = b % XCDS, j = b / XCDS;
    const int q = total / XCDS, rmd = total % XCDS;
    tile_of_item(x * q + min(x, rmd) + j, offsets, tprefix, G, nrows, BM, NT, MT, tc, nsup);
    return true;
}

// Balanced schedule.  The XCDs of one launch run at different shader clocks
// (measured per XCD with s_memtime: up to ~10 % apart under the GEMMs' load), so
// equal static runs leave the fast XCDs idle at the end.  Each XCD's run keeps
// its first 7/8 static (taken by workgroup index, as in tile_coords); the last
// eighth is claimed at run time.  Per XCD one 64-bit counter q[x] holds (low
// half) the items its own workgroups took from the front of that eighth and
// (high half) the items other XCDs' workgroups took from its back.  A claim is
// one atomic add that returns both counts: it is valid iff their sum was below
// the eighth's length D, which makes front and back claims disjoint and the
// first D claims cover the eighth exactly.  A workgroup past its own eighth
// steals from the back of the XCD with the most items left; a failed steal
// leaves that XCD with none left for good, so at most 8 attempts are made.
// The grid's workgroups past the item count (the host sizes the grid for the
// largest possible tile count) are extra claimers, so a fast XCD can take more
// than its own eighth.  Returns the item, or -1 when every item is taken.
// Executed by all threads of the workgroup (the branch is uniform); `bcast` is
// LDS the workgroup may use.
__device__ __forceinline__ int claim_item(int b, int total, unsigned long long* __restrict__ q, int* bcast) {
    const int x = b % XCDS, j = b / XCDS;
    const int qq = total / XCDS, rmd = total % XCDS;
    const int Lx = qq + (x < rmd ? 1 : 0), start = x * qq + min(x, rmd);
    const int Sx = Lx - (Lx >> 3);
    if (j < Sx) return start + j;
    if (total == 0) return -1;
    if (threadIdx.x == 0) {
        int w = -1;
        if (j < Lx) {   // one of the run's own workgroups: the front of its eighth first
            const unsigned long long o =
                __hip_atomic_fetch_add(q + x, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int h = (int)(o & 0xffffffffull), t = (int)(o >> 32);
            if (h + t < (Lx >> 3)) w = start + Sx + h;
        }
        // workgroups past the run (the grid's slack) go straight to stealing
        for (int attempt = 0; attempt <= XCDS && w < 0; ++attempt) {
            int best = -1, left = 0;
            for (int y = 0; y < XCDS; ++y) {
                const unsigned long long v = __hip_atomic_load(q + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int Dy = (qq + (y < rmd ? 1 : 0)) >> 3;
                const int r = Dy - (int)(v & 0xffffffffull) - (int)(v >> 32);
                if (r > left) {
                    left = r;
                    best = y;
                }
            }
            if (best < 0) break;
            const unsigned long long v =
                __hip_atomic_fetch_add(q + best, 1ull << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int Ly = qq + (best < rmd ? 1 : 0), Dy = Ly >> 3;
            const int hy = (int)(v & 0xffffffffull), ty = (int)(v >> 32);
            if (hy + ty < Dy) w = best * qq + min(best, rmd) + (Ly - Dy) + (Dy - 1 - ty);
        }
        *bcast = w;
    }
    __syncthreads();
    const int w = *bcast;
    __syncthreads();   // the word is overwritten by the first tile loads
    return w;
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
    if (g < MOE_SCHED_WORDS) moe_sched_words(tprefix, G)[g] = 0ull;
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
// helpers of the scheduled bf16 kernel
// ---------------------------------------------------------------------------

// gfx950's direct global->LDS load (16 bytes per lane to M0 + 16 * lane) issued
// from a tiny asm statement.  It has no
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
        "s_nop 0\n\t"   // one wait state between the M0 write and the LDS-DMA load
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_wave_addr)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

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


// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM: 8 waves, global->LDS ring, one scheduled asm block per K tile
// ---------------------------------------------------------------------------
//
// Workgroup tile 256 rows x BN output columns (GEMM1: BN = 128 gate + 128 up
// weight rows in one B tile; GEMM2: BN = 256), 8 waves = 2 per SIMD in a 4 x 2
// grid, each wave owning 64 rows x 4 B fragments of 32 columns (8 accumulators of
// 32x32, held in AGPRs).  K advances in tiles of 64 through LDS: two 32 KB
// activation stages and three 32 KB weight stages (all 160 KB), filled by
// gfx950's direct global->LDS loads (8 per wave per tile, one full 128-byte
// line per row segment); the weights, the operand streamed from HBM, run two K
// tiles ahead.
//
// The steady-state K tile is one asm block with a fixed instruction order; the
// compiler, left to itself, reuses operand registers and serialises LDS reads
// with the MFMAs that consume them.  Per substep of K 16 the wave waits for its
// operands, then alternates one MFMA with one LDS read of the next substep's
// operands; the first substep also issues the 4 weight loads of tile kt + 2 (into
// the weight stage tile kt - 1 used).  Before the last substep the wave waits for
// its own loads of the next tile (the newest 4, those weights, may stay in
// flight) and meets the other waves at a barrier (after which the activation
// stage just consumed is free), then alternates the last MFMAs with the 4
// activation loads of tile kt + 2 and the reads of the next tile's first
// operands.  Splitting the 8 loads over two substeps instead of one burst saved
// ~3 % of the layer.  Every LDS read the block issues is waited for inside the
// block.  Past the barrier a wave raises its issue priority (s_setprio 1) and
// drops it again after the next tile's first substep, so the waves still in
// that stretch -- the ones behind -- win the SIMD's issue over those already
// past it and the workgroup reaches its next barrier closer together (GEMM1
// of the Mixtral layer 2.5-3.5 % faster, GEMM2 ~2 %, same-box A/B; raising it
// in steps over all four substeps measured the same).
//
// The MFMAs take the weight fragment as their first operand (C^T = B^T A^T), so a
// lane's accumulator holds one output row and, per group of 4 registers, 4
// consecutive output columns: the epilogue stores 8 (bf16) or 16 (fp32) bytes
// per lane and group.  Each output element is still the same fp32 sum over k in
// the same order.

#define MOE_MF(c, a, b) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #b "], %[" #a "], %[" #c "]\n\t"
#define MOE_DSR(dst, addr, off) "ds_read_b128 %[" #dst "], %[" #addr "] offset:" off "\n\t"
#define MOE_DSRI(dst, addr, off) "ds_read_b128 %[" #dst "], %[" #addr "] offset:%[" #off "]\n\t"
// A load's M0 (LDS destination) is written one instruction or more before the
// load itself: the ISA requires a wait state between the two.
#define MOE_M0(lds, imm) "s_add_u32 m0, %[" #lds "], " imm "\n\t"
#define MOE_LD(vo, sb) "global_load_lds_dwordx4 %[" #vo "], %[" #sb "]\n\t"
#define MOE_DMA(vo, sb, lds, imm) MOE_M0(lds, imm) "s_nop 0\n\t" MOE_LD(vo, sb)
// One substep: multiply operand set P (A fragments a0 a1, B fragments b0..b3) while
// reading the next substep into Q (in the order a0 b0 a1 b1 b2 b3).
#define MOE_SUBSTEP(P, Q, RA, RB)                                 \
    "s_waitcnt lgkmcnt(0)\n\t"                                    \
    MOE_MF(c0, P##a0, P##b0) MOE_DSR(Q##a0, RA, "0")              \
    MOE_MF(c1, P##a1, P##b0) MOE_DSR(Q##b0, RB, "0")              \
    MOE_MF(c2, P##a0, P##b1) MOE_DSR(Q##a1, RA, "4096")           \
    MOE_MF(c3, P##a1, P##b1) MOE_DSRI(Q##b1, RB, ob1)             \
    MOE_MF(c4, P##a0, P##b2) MOE_DSRI(Q##b2, RB, ob2)             \
    MOE_MF(c5, P##a1, P##b2) MOE_DSRI(Q##b3, RB, ob3)             \
    MOE_MF(c6, P##a0, P##b3)                                      \
    MOE_MF(c7, P##a1, P##b3)
// First substep of a block: as MOE_SUBSTEP, with this block's 4 weight-tile
// loads (into the weight stage freed by the previous block's barrier) between
// the MFMAs.
#define MOE_SUBSTEP_B(P, Q, RA, RB)                                                      \
    "s_waitcnt lgkmcnt(0)\n\t"                                                           \
    MOE_M0(ldsB, "0") MOE_MF(c0, P##a0, P##b0) MOE_LD(vo4, sb0) MOE_DSR(Q##a0, RA, "0")  \
    MOE_M0(ldsB, "8192") MOE_MF(c1, P##a1, P##b0) MOE_LD(vo5, sb1) MOE_DSR(Q##b0, RB, "0") \
    MOE_M0(ldsB, "16384") MOE_MF(c2, P##a0, P##b1) MOE_LD(vo6, sb2) MOE_DSR(Q##a1, RA, "4096") \
    MOE_M0(ldsB, "24576") MOE_MF(c3, P##a1, P##b1) MOE_LD(vo7, sb3) MOE_DSRI(Q##b1, RB, ob1) \
    MOE_MF(c4, P##a0, P##b2) MOE_DSRI(Q##b2, RB, ob2)                                    \
    MOE_MF(c5, P##a1, P##b2) MOE_DSRI(Q##b3, RB, ob3)                                    \
    MOE_MF(c6, P##a0, P##b3)                                                             \
    MOE_MF(c7, P##a1, P##b3)
#define MOE_SUBSTEP_HALF_B(P, Q, RA, RB)                                                 \
    "s_waitcnt lgkmcnt(0)\n\t"                                                           \
    MOE_M0(ldsB, "0") MOE_MF(c0, P##a0, P##b0) MOE_LD(vo4, sb0) MOE_DSR(Q##a0, RA, "0")  \
    MOE_M0(ldsB, "8192") MOE_MF(c2, P##a0, P##b1) MOE_LD(vo5, sb1) MOE_DSR(Q##b0, RB, "0") \
    MOE_M0(ldsB, "16384") MOE_MF(c4, P##a0, P##b2) MOE_LD(vo6, sb2) MOE_DSRI(Q##b1, RB, ob1) \
    MOE_M0(ldsB, "24576") MOE_MF(c6, P##a0, P##b3) MOE_LD(vo7, sb3) MOE_DSRI(Q##b2, RB, ob2) \
    MOE_DSRI(Q##b3, RB, ob3)
#define MOE_LASTSUB                                                                      \
    "s_waitcnt lgkmcnt(0)\n\t"                                                           \
    "s_waitcnt vmcnt(4)\n\t"                                                             \
    "s_barrier\n\t"                                                                      \
    "s_setprio 1\n\t"                                                                     \
    MOE_M0(ldsA, "0") MOE_MF(c0, ya0, yb0) MOE_LD(vo0, sa)                                  \
    MOE_M0(ldsA, "8192") MOE_MF(c1, ya1, yb0) MOE_LD(vo1, sa) MOE_DSR(xa0, na0, "0")        \
    MOE_M0(ldsA, "16384") MOE_MF(c2, ya0, yb1) MOE_LD(vo2, sa) MOE_DSR(xb0, nb0, "0")       \
    MOE_M0(ldsA, "24576") MOE_MF(c3, ya1, yb1) MOE_LD(vo3, sa) MOE_DSR(xa1, na0, "4096")    \
    MOE_MF(c4, ya0, yb2) MOE_DSRI(xb1, nb0, ob1)                                         \
    MOE_MF(c5, ya1, yb2) MOE_DSRI(xb2, nb0, ob2)                                         \
    MOE_MF(c6, ya0, yb3) MOE_DSRI(xb3, nb0, ob3)                                         \
    MOE_MF(c7, ya1, yb3)                                                                 \
    "s_waitcnt lgkmcnt(0)\n\t"

// One steady-state K tile.  x: operands of substep 0 of this tile on entry, of
// the next tile on exit.  ra*/rb*: LDS byte addresses of the A / B fragment 0 of
// substeps 1..3 of this tile; na0/nb0: of substep 0 of the next tile.  OB1..3:
// byte offsets of B fragments 1..3.  vo: per-lane byte offsets of the 8 refill
// loads from the SGPR bases sa (A) and sb0..3 (B) of tile kt + 2; ldsA/ldsB:
// this wave's LDS destination of load 0 in the stage being refilled (load i lands
// 8 KB further on).
template <int OB1, int OB2, int OB3>
__device__ __forceinline__ void gemm_tile_asm(floatx16_t (&c)[8], bf16x8_t (&x)[6], uint32_t ra1, uint32_t rb1,
                                              uint32_t ra2, uint32_t rb2, uint32_t ra3, uint32_t rb3,
                                              uint32_t na0, uint32_t nb0, const uint32_t (&vo)[8], const void* sa,
                                              const void* sb0, const void* sb1, const void* sb2, const void* sb3,
                                              uint32_t ldsA, uint32_t ldsB) {
    bf16x8_t y[6];
    uint32_t saved_m0;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 MOE_SUBSTEP_B(x, y, ra1, rb1)
                 "s_setprio 0\n\t"
                 MOE_SUBSTEP(y, x, ra2, rb2)
                 MOE_SUBSTEP(x, y, ra3, rb3)
                 MOE_LASTSUB
                 "s_mov_b32 m0, %[sv]"
                 : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [c4] "+a"(c[4]),
                   [c5] "+a"(c[5]), [c6] "+a"(c[6]), [c7] "+a"(c[7]), [xa0] "+v"(x[0]), [xa1] "+v"(x[1]),
                   [xb0] "+v"(x[2]), [xb1] "+v"(x[3]), [xb2] "+v"(x[4]), [xb3] "+v"(x[5]), [ya0] "=&v"(y[0]),
                   [ya1] "=&v"(y[1]), [yb0] "=&v"(y[2]), [yb1] "=&v"(y[3]), [yb2] "=&v"(y[4]), [yb3] "=&v"(y[5]),
                   [sv] "=&s"(saved_m0)
                 : [ra1] "v"(ra1), [rb1] "v"(rb1), [ra2] "v"(ra2), [rb2] "v"(rb2), [ra3] "v"(ra3), [rb3] "v"(rb3),
                   [na0] "v"(na0), [nb0] "v"(nb0), [ob1] "i"(OB1), [ob2] "i"(OB2), [ob3] "i"(OB3),
                   [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3]), [vo4] "v"(vo[4]),
                   [vo5] "v"(vo[5]), [vo6] "v"(vo[6]), [vo7] "v"(vo[7]), [sa] "s"(sa), [sb0] "s"(sb0),
                   [sb1] "s"(sb1), [sb2] "s"(sb2), [sb3] "s"(sb3), [ldsA] "s"(ldsA), [ldsB] "s"(ldsB)
                 : "memory");
}

// Waves whose 64 rows hold at most 32 valid ones run only the MFMAs of A fragment 0
// (and read no A fragment 1); waves with no valid row run no MFMA and read
// nothing.  Both still issue their share of the refill loads and meet the same
// barrier, so the workgroup's load plan and synchronisation are unchanged.
#define MOE_SUBSTEP_HALF(P, Q, RA, RB)                            \
    "s_waitcnt lgkmcnt(0)\n\t"                                    \
    MOE_MF(c0, P##a0, P##b0) MOE_DSR(Q##a0, RA, "0")              \
    MOE_MF(c2, P##a0, P##b1) MOE_DSR(Q##b0, RB, "0")              \
    MOE_MF(c4, P##a0, P##b2) MOE_DSRI(Q##b1, RB, ob1)             \
    MOE_MF(c6, P##a0, P##b3) MOE_DSRI(Q##b2, RB, ob2)             \
    MOE_DSRI(Q##b3, RB, ob3)
#define MOE_LASTSUB_HALF                                                                 \
    "s_waitcnt lgkmcnt(0)\n\t"                                                           \
    "s_waitcnt vmcnt(4)\n\t"                                                             \
    "s_barrier\n\t"                                                                      \
    "s_setprio 1\n\t"                                                                     \
    MOE_M0(ldsA, "0") MOE_MF(c0, ya0, yb0) MOE_LD(vo0, sa)                                  \
    MOE_M0(ldsA, "8192") MOE_DSR(xa0, na0, "0") MOE_LD(vo1, sa)                             \
    MOE_M0(ldsA, "16384") MOE_MF(c2, ya0, yb1) MOE_LD(vo2, sa)                              \
    MOE_M0(ldsA, "24576") MOE_DSR(xb0, nb0, "0") MOE_LD(vo3, sa)                            \
    MOE_MF(c4, ya0, yb2) MOE_DSRI(xb1, nb0, ob1) MOE_DSRI(xb2, nb0, ob2)                 \
    MOE_MF(c6, ya0, yb3) MOE_DSRI(xb3, nb0, ob3)                                         \
    "s_waitcnt lgkmcnt(0)\n\t"

template <int OB1, int OB2, int OB3>
__device__ __forceinline__ void gemm_tile_asm_half(floatx16_t (&c)[8], bf16x8_t (&x)[6], uint32_t ra1, uint32_t rb1,
                                                   uint32_t ra2, uint32_t rb2, uint32_t ra3, uint32_t rb3,
                                                   uint32_t na0, uint32_t nb0, const uint32_t (&vo)[8],
                                                   const void* sa, const void* sb0, const void* sb1,
                                                   const void* sb2, const void* sb3, uint32_t ldsA, uint32_t ldsB) {
    bf16x8_t y[6];
    uint32_t saved_m0;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 MOE_SUBSTEP_HALF_B(x, y, ra1, rb1)
                 "s_setprio 0\n\t"
                 MOE_SUBSTEP_HALF(y, x, ra2, rb2)
                 MOE_SUBSTEP_HALF(x, y, ra3, rb3)
                 MOE_LASTSUB_HALF
                 "s_mov_b32 m0, %[sv]"
                 : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [c4] "+a"(c[4]),
                   [c5] "+a"(c[5]), [c6] "+a"(c[6]), [c7] "+a"(c[7]), [xa0] "+v"(x[0]), [xa1] "+v"(x[1]),
                   [xb0] "+v"(x[2]), [xb1] "+v"(x[3]), [xb2] "+v"(x[4]), [xb3] "+v"(x[5]), [ya0] "=&v"(y[0]),
                   [ya1] "=&v"(y[1]), [yb0] "=&v"(y[2]), [yb1] "=&v"(y[3]), [yb2] "=&v"(y[4]), [yb3] "=&v"(y[5]),
                   [sv] "=&s"(saved_m0)
                 : [ra1] "v"(ra1), [rb1] "v"(rb1), [ra2] "v"(ra2), [rb2] "v"(rb2), [ra3] "v"(ra3), [rb3] "v"(rb3),
                   [na0] "v"(na0), [nb0] "v"(nb0), [ob1] "i"(OB1), [ob2] "i"(OB2), [ob3] "i"(OB3),
                   [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3]), [vo4] "v"(vo[4]),
                   [vo5] "v"(vo[5]), [vo6] "v"(vo[6]), [vo7] "v"(vo[7]), [sa] "s"(sa), [sb0] "s"(sb0),
                   [sb1] "s"(sb1), [sb2] "s"(sb2), [sb3] "s"(sb3), [ldsA] "s"(ldsA), [ldsB] "s"(ldsB)
                 : "memory");
}

__device__ __forceinline__ void gemm_tile_asm_loads_only(floatx16_t (&c)[8], bf16x8_t (&x)[6], const uint32_t (&vo)[8],
                                                         const void* sa, const void* sb0, const void* sb1,
                                                         const void* sb2, const void* sb3, uint32_t ldsA,
                                                         uint32_t ldsB) {
    uint32_t saved_m0;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 MOE_DMA(vo4, sb0, ldsB, "0") MOE_DMA(vo5, sb1, ldsB, "8192")
                 MOE_DMA(vo6, sb2, ldsB, "16384") MOE_DMA(vo7, sb3, ldsB, "24576")
                 "s_waitcnt vmcnt(4)\n\t"
                 "s_barrier\n\t"
                 MOE_DMA(vo0, sa, ldsA, "0") MOE_DMA(vo1, sa, ldsA, "8192") MOE_DMA(vo2, sa, ldsA, "16384")
                 MOE_DMA(vo3, sa, ldsA, "24576")
                 "s_mov_b32 m0, %[sv]"
                 : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [c4] "+a"(c[4]),
                   [c5] "+a"(c[5]), [c6] "+a"(c[6]), [c7] "+a"(c[7]), [xa0] "+v"(x[0]), [xa1] "+v"(x[1]),
                   [xb0] "+v"(x[2]), [xb1] "+v"(x[3]), [xb2] "+v"(x[4]), [xb3] "+v"(x[5]), [sv] "=&s"(saved_m0)
                 : [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3]), [vo4] "v"(vo[4]),
                   [vo5] "v"(vo[5]), [vo6] "v"(vo[6]), [vo7] "v"(vo[7]), [sa] "s"(sa), [sb0] "s"(sb0),
                   [sb1] "s"(sb1), [sb2] "s"(sb2), [sb3] "s"(sb3), [ldsA] "s"(ldsA), [ldsB] "s"(ldsB)
                 : "memory");
}

// Thin tiles: the last row tile of a group that also has full tiles, holding at
// most 64 valid rows.  Its weight tiles are the ones its sibling tiles read at
// about the same time, so they mostly hit in L2 and the K loop is bound by load
// latency, not bandwidth: it gets a deeper prefetch.  (A group of at most 64 rows
// in all streams its weights from HBM alone; there the standard pipeline was as
// fast, and faster for the layer as a whole, so it keeps it.)  The rows are split
// into two 32-row halves over the waves of A row slots 0 and 1, so four waves on
// four SIMDs each run the A-fragment-0 MFMAs; the others only load.
// An activation tile needs just 8 KB, so the activation stages become four 8 KB
// slots and the freed 32 KB holds a fourth weight stage: both operands stream
// three K tiles ahead.  Block kt loads the weights of kt + 3 in its first substep
// and the activations of kt + 3 (one load per wave) in its second; at its barrier
// the wave's loads of tile kt + 1 are complete when at most the 10 issued after
// them (tiles kt + 2 and kt + 3) are in flight.
#define MOE_SUBSTEP_HALF_A1(P, Q, RA, RB)                                                \
    "s_waitcnt lgkmcnt(0)\n\t"                                                           \
    MOE_M0(ldsA, "0") MOE_MF(c0, P##a0, P##b0) MOE_LD(vo0, sa) MOE_DSR(Q##a0, RA, "0")   \
    MOE_MF(c2, P##a0, P##b1) MOE_DSR(Q##b0, RB, "0")                                     \
    MOE_MF(c4, P##a0, P##b2) MOE_DSRI(Q##b1, RB, ob1)                                    \
    MOE_MF(c6, P##a0, P##b3) MOE_DSRI(Q##b2, RB, ob2)                                    \
    MOE_DSRI(Q##b3, RB, ob3)
#define MOE_LASTSUB_HALF_THIN                                                            \
    "s_waitcnt lgkmcnt(0)\n\t"                                                           \
    "s_waitcnt vmcnt(10)\n\t"                                                            \
    "s_barrier\n\t"                                                                      \
    "s_setprio 1\n\t"                                                                     \
    MOE_MF(c0, ya0, yb0) MOE_DSR(xa0, na0, "0")                                          \
    MOE_MF(c2, ya0, yb1) MOE_DSR(xb0, nb0, "0")                                          \
    MOE_MF(c4, ya0, yb2) MOE_DSRI(xb1, nb0, ob1) MOE_DSRI(xb2, nb0, ob2)                 \
    MOE_MF(c6, ya0, yb3) MOE_DSRI(xb3, nb0, ob3)                                         \
    "s_waitcnt lgkmcnt(0)\n\t"

template <int OB1, int OB2, int OB3>
__device__ __forceinline__ void gemm_tile_asm_thin(floatx16_t (&c)[8], bf16x8_t (&x)[6], uint32_t ra1, uint32_t rb1,
                                                   uint32_t ra2, uint32_t rb2, uint32_t ra3, uint32_t rb3,
                                                   uint32_t na0, uint32_t nb0, const uint32_t (&vo)[8],
                                                   const void* sa, const void* sb0, const void* sb1,
                                                   const void* sb2, const void* sb3, uint32_t ldsA, uint32_t ldsB) {
    bf16x8_t y[6];
    uint32_t saved_m0;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 MOE_SUBSTEP_HALF_B(x, y, ra1, rb1)
                 "s_setprio 0\n\t"
                 MOE_SUBSTEP_HALF_A1(y, x, ra2, rb2)
                 MOE_SUBSTEP_HALF(x, y, ra3, rb3)
                 MOE_LASTSUB_HALF_THIN
                 "s_mov_b32 m0, %[sv]"
                 : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [c4] "+a"(c[4]),
                   [c5] "+a"(c[5]), [c6] "+a"(c[6]), [c7] "+a"(c[7]), [xa0] "+v"(x[0]), [xa1] "+v"(x[1]),
                   [xb0] "+v"(x[2]), [xb1] "+v"(x[3]), [xb2] "+v"(x[4]), [xb3] "+v"(x[5]), [ya0] "=&v"(y[0]),
                   [ya1] "=&v"(y[1]), [yb0] "=&v"(y[2]), [yb1] "=&v"(y[3]), [yb2] "=&v"(y[4]), [yb3] "=&v"(y[5]),
                   [sv] "=&s"(saved_m0)
                 : [ra1] "v"(ra1), [rb1] "v"(rb1), [ra2] "v"(ra2), [rb2] "v"(rb2), [ra3] "v"(ra3), [rb3] "v"(rb3),
                   [na0] "v"(na0), [nb0] "v"(nb0), [ob1] "i"(OB1), [ob2] "i"(OB2), [ob3] "i"(OB3),
                   [vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3]), [vo4] "v"(vo[4]),
                   [vo5] "v"(vo[5]), [vo6] "v"(vo[6]), [vo7] "v"(vo[7]), [sa] "s"(sa), [sb0] "s"(sb0),
                   [sb1] "s"(sb1), [sb2] "s"(sb2), [sb3] "s"(sb3), [ldsA] "s"(ldsA), [ldsB] "s"(ldsB)
                 : "memory");
}

__device__ __forceinline__ void gemm_tile_asm_loads_only_thin(floatx16_t (&c)[8], bf16x8_t (&x)[6],
                                                              const uint32_t (&vo)[8], const void* sa,
                                                              const void* sb0, const void* sb1, const void* sb2,
                                                              const void* sb3, uint32_t ldsA, uint32_t ldsB) {
    uint32_t saved_m0;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 MOE_DMA(vo4, sb0, ldsB, "0") MOE_DMA(vo5, sb1, ldsB, "8192")
                 MOE_DMA(vo6, sb2, ldsB, "16384") MOE_DMA(vo7, sb3, ldsB, "24576")
                 MOE_DMA(vo0, sa, ldsA, "0")
                 "s_waitcnt vmcnt(10)\n\t"
                 "s_barrier\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [c0] "+a"(c[0]), [c1] "+a"(c[1]), [c2] "+a"(c[2]), [c3] "+a"(c[3]), [c4] "+a"(c[4]),
                   [c5] "+a"(c[5]), [c6] "+a"(c[6]), [c7] "+a"(c[7]), [xa0] "+v"(x[0]), [xa1] "+v"(x[1]),
                   [xb0] "+v"(x[2]), [xb1] "+v"(x[3]), [xb2] "+v"(x[4]), [xb3] "+v"(x[5]), [sv] "=&s"(saved_m0)
                 : [vo0] "v"(vo[0]), [vo4] "v"(vo[4]), [vo5] "v"(vo[5]), [vo6] "v"(vo[6]), [vo7] "v"(vo[7]),
                   [sa] "s"(sa), [sb0] "s"(sb0), [sb1] "s"(sb1), [sb2] "s"(sb2), [sb3] "s"(sb3), [ldsA] "s"(ldsA),
                   [ldsB] "s"(ldsB)
                 : "memory");
}

// Requires K % 64 == 0, N % 8 == 0 and 512 K < 2^32 (32-bit load offsets).
// K split: the grid is S copies of a tile grid of gridDim.x / S workgroups (a
// multiple of 8, so every copy keeps the XCD order); copy s sums the K tiles
// [s KT / S, (s + 1) KT / S) of the KT = K / 64 and writes its fp32 partial to
// Cout (s = 0) or Cpart + (s - 1) part_stride (s >= 1).  SwiGLU with S > 1
// writes the fp32 gate and up partials instead (see swiglu_part), and
// swiglu_reduce_kernel forms h from them.
template <int BN, bool SWIGLU, bool SPLIT_GU = false>
__global__ __launch_bounds__(512, 1) void gemm_bf16_asm_kernel(const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ B0,
                                                               const uint16_t* __restrict__ B1,
                                                               void* __restrict__ Cout, float* __restrict__ Cpart,
                                                               int64_t part_stride,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ tprefix, int G,
                                                               int64_t nrows, int N, int K, int S, int nsup,
                                                               int thin_all, const int32_t* __restrict__ gather,
                                                               unsigned long long* __restrict__ sched) {
    constexpr int BM = 256, BK = 64, WGN = 2, WAVES = 8;
    constexpr int NOPS = SWIGLU ? 2 : 1;
    constexpr int WM = 64, WN = BN / WGN;       // wave tile: 64 rows x WN columns of each operand
    constexpr int NTW = WN / 32;                // B fragments per operand per wave
    static_assert(NOPS * NTW == 4, "4 B fragments per wave");
    constexpr int STAGE = BM * BK * 2;          // bytes of one operand stage (256 rows x 64 bf16)
    // B fragment f = (operand o, j) starts at B tile row o * BN + j * 32 (plus the wave's offset)
    constexpr int OB1 = 32 * 128;
    constexpr int OB2 = (NOPS == 2 ? BN : 64) * 128;
    constexpr int OB3 = (NOPS == 2 ? BN + 32 : 96) * 128;
    constexpr int OBF[4] = {0, OB1, OB2, OB3};

    // activation K tiles: 2 stages, then weight K tiles: 3 stages (all 160 KB of LDS)
    __shared__ uint4 lds[5 * STAGE / 16];
    uint4* const sA = lds;
    uint4* const sB = lds + 2 * STAGE / 16;

    TileCoord tc;
    const int NT = (N + BN - 1) / BN;
    const int tiles_grid = gridDim.x / S;
    const int split = blockIdx.x / tiles_grid;
    if (sched && split == S - 1) {
        // balanced schedule for the last K-split copy, whose end is the launch's
        // end (earlier copies are followed by the next copy's work, and their grid
        // slack is dispatched mid-launch, too early to balance anything); the LDS
        // word is free until the first tile loads
        const int MT = tile_count(offsets, tprefix, G, nrows, BM);
        const int b = blockIdx.x - split * tiles_grid;
        const int w = claim_item(b, MT * NT, sched, reinterpret_cast<int*>(lds));
        if (w < 0) return;
        tile_of_item(w, offsets, tprefix, G, nrows, BM, NT, MT, tc, nsup);
    } else if (!tile_coords(blockIdx.x - split * tiles_grid, offsets, tprefix, G, nrows, BM, NT, tc, nsup)) {
        return;
    }
    const int KTall = K / BK;
    const int kt_begin = split * KTall / S, kt_end = (split + 1) * KTall / S;
    // SPLIT_GU (SwiGLU, S > 1): fp32 gate / up partials, gate of split s at Cpart + s
    // part_stride, up at Cpart + (S + s) part_stride; otherwise split 0 writes Cout
    // and split s >= 1 its fp32 partial at Cpart + (s - 1) part_stride.
    constexpr bool swiglu_part = SWIGLU && SPLIT_GU;
    void* C = split ? static_cast<void*>(Cpart + (int64_t)(split - 1) * part_stride) : Cout;

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm = wave / WGN, wn = wave % WGN;
    // thin: a last row tile of <= 64 rows behind full tiles of the same group
    // (thin_all: every tile of <= 64 rows, for launches whose whole grid is one
    // round of workgroups — small batches, where each CU streams one tile)
    const bool thin = tc.row_end - tc.row_start <= 64 &&
                      (thin_all || tc.row_start > (offsets ? offsets[tc.g] : 0));
    const int arow = thin ? 32 * wm : WM * wm;   // first tile row of this wave's A fragment 0
    const int n0 = tc.nt * BN;
    const int64_t wstride = (int64_t)N * K;
    const int64_t k0 = (int64_t)kt_begin * BK;
    const uint16_t* Bg = B0 + (int64_t)tc.g * wstride + (int64_t)n0 * K + k0;
    const uint16_t* Bu = SWIGLU ? B1 + (int64_t)tc.g * wstride + (int64_t)n0 * K + k0 : Bg;
    const uint16_t* At = A + (gather ? 0 : tc.row_start * K) + k0;

    // Load plan: load i of wave w fills tile rows (8 i + w) * 8 + lane / 8 at
    // physical chunk lane % 8, i.e. logical chunk (lane % 8) ^ swz(row).  A rows
    // past the group end and weight rows past N read tile row 0 instead (their
    // outputs are never stored).  Offsets are bytes from At / the weight base.
    // gather (nullable): tile row r is row gather[row_start + r] of A (the grouped
    // rows are read in place from the token-ordered activations); the indices of a
    // wave's 8 consecutive rows are one scalar load, so no vector-memory wait
    // stands before the first tile loads.
    uint32_t vo[8];
    const uint16_t* bbase[4];
    int32_t gv[4][8] = {}, g0 = 0;
    if (gather) {   // all index loads first (uniform addresses), then one wait
        g0 = __builtin_amdgcn_readfirstlane(gather[tc.row_start]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                gv[i][j] = __builtin_amdgcn_readfirstlane(gather[tc.row_start + (WAVES * i + wave) * 8 + j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (WAVES * i + wave) * 8 + lane / 8;
        const int ch = (lane % 8) ^ lds_swz(row);
        const bool ok = tc.row_start + row < tc.row_end;
        int64_t src = ok ? row : 0;
        if (gather) {
            int32_t mine = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) mine = lane / 8 == j ? gv[i][j] : mine;
            src = ok ? mine : g0;
        }
        vo[i] = (uint32_t)((src * K + ch * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (WAVES * i + wave) * 8 + lane / 8;   // B tile row
        const int op = row / BN, rr = row % BN;
        const int ch = (lane % 8) ^ lds_swz(row);
        const int r = n0 + rr < N ? rr : 0;
        vo[4 + i] = (uint32_t)(((int64_t)r * K + ch * 8) * 2);
        bbase[i] = op ? Bu : Bg;
    }
    const uint32_t sA_addr = lds_byte_addr(sA), sB_addr = lds_byte_addr(sB);
    auto load_a = [&](int kt, int stage) {
        const uint32_t la = sA_addr + stage * STAGE + wave * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_async(At + (int64_t)kt * BK + vo[i] / 2, la + i * 8192);
    };
    auto load_b = [&](int kt, int stage) {
        const uint32_t lb = sB_addr + stage * STAGE + wave * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_async(bbase[i] + (int64_t)kt * BK + vo[4 + i] / 2, lb + i * 8192);
    };
    // thin tiles: activation tile t in 8 KB slot t % 4; weight stage 3 is the upper
    // half of the activation area (byte offset from weight stage 0: -STAGE)
    auto thin_boff = [&](int t) -> int { return (t & 3) == 3 ? -STAGE : (t & 3) * STAGE; };
    auto load_a_thin = [&](int kt, int t) {
        dma16_async(At + (int64_t)kt * BK + vo[0] / 2, sA_addr + (t & 3) * 8192 + wave * 1024);
    };
    auto load_b_thin = [&](int kt, int t) {
        const uint32_t lb = sB_addr + thin_boff(t) + wave * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_async(bbase[i] + (int64_t)kt * BK + vo[4 + i] / 2, lb + i * 8192);
    };

    floatx16_t c[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v) c[q][v] = 0.f;

    // K tile kt lives in activation stage kt % 2 and weight stage kt % 3.  Block
    // kt loads the weights of kt + 2 in its first substep and the activations of
    // kt + 2 after its barrier, so weights stream ~2 tiles ahead.  Thin tiles:
    // activation slot kt % 4, weight stage kt % 4, both loaded 3 tiles ahead.
    const int KT = kt_end - kt_begin;
    if (thin) {
        // tiles 0..2 of both operands (indices past the end reload the last tile
        // into a slot nobody reads, so the wait counts below always hold)
        for (int t = 0; t < 3; ++t) {
            load_b_thin(min(t, KT - 1), t);
            load_a_thin(min(t, KT - 1), t);
        }
    } else {
        load_a(0, 0);
        load_b(0, 0);
        if (KT > 1) {
            load_a(1, 1);
            load_b(1, 1);
        }
    }

    const int lrow = lane % 32, lhalf = lane / 32;
    const int rswz = lds_swz(lrow);
    // LDS byte address of fragment 0 of substep s in stage 0 (32 rows per fragment: A
    // fragment 1 is 4096 bytes on, B fragments at OBF)
    uint32_t ra[4], rb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cc = (2 * s + lhalf) ^ rswz;
        ra[s] = sA_addr + ((arow + lrow) * 8 + cc) * 16;   // arow % 16 == 0: same swizzle
        rb[s] = sB_addr + ((wn * WN + lrow) * 8 + cc) * 16;
    }
    // aoff / boff: byte offset of the stage from activation / weight stage 0
    auto read_sub = [&](int aoff, int boff, int s, bf16x8_t (&o)[6]) {
        const char* base = reinterpret_cast<const char*>(lds);
        const char* pa = base + (int)(ra[s] - sA_addr) + aoff;
        const char* pb = base + (int)(rb[s] - sA_addr) + boff;
        o[0] = as_bf16x8(*reinterpret_cast<const uint4*>(pa));
        o[1] = as_bf16x8(*reinterpret_cast<const uint4*>(pa + 4096));
#pragma unroll
        for (int f = 0; f < 4; ++f) o[2 + f] = as_bf16x8(*reinterpret_cast<const uint4*>(pb + OBF[f]));
    };
    auto aoff_of = [&](int t) -> int { return thin ? (t & 3) * 8192 : (t & 1) * STAGE; };
    auto boff_of = [&](int t) -> int { return thin ? thin_boff(t) : (t % 3) * STAGE; };
    // valid rows of this wave's 64: > 32 -> all MFMAs, 1..32 -> A fragment 0 only, 0 -> none
    // (thin tiles: 32 rows per wave, so never more than A fragment 0)
    const int64_t wave_rows = tc.row_end - (tc.row_start + arow);
    const int mode = thin ? (wave_rows > 0 ? 1 : 0) : (wave_rows > 32 ? 2 : (wave_rows > 0 ? 1 : 0));
    // accumulator q = (A fragment q % 2, B fragment q / 2); weight fragment first (C^T)
    auto mma = [&](const bf16x8_t (&o)[6]) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            c[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[2 + q / 2], o[q % 2], c[q], 0, 0, 0);
    };

    // tile 0 must have landed; the loads issued after it may still be in flight
    if (thin) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else if (KT > 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier_reads_done();
    bf16x8_t x[6];
    read_sub(0, 0, 0, x);
    // steady state: one loop per wave mode (the mode is uniform across the wave)
    int kt = 0, sb = 0;   // sb = kt % 3
    if (thin) {
        // every block but the last; loads past the last tile reload it into a free slot
#define MOE_THIN_ARGS(kt_)                                                                              \
    const uint32_t so = ((kt_) & 3) * 8192, no = (((kt_) + 1) & 3) * 8192;                              \
    const uint32_t sbo = (uint32_t)thin_boff(kt_), nbo = (uint32_t)thin_boff((kt_) + 1);                \
    const int64_t koff = (int64_t)min((kt_) + 3, KT - 1) * BK;                                          \
    const uint32_t ldsA = sA_addr + (((kt_) + 3) & 3) * 8192 + wave * 1024;                             \
    const uint32_t ldsB = sB_addr + (uint32_t)thin_boff((kt_) + 3) + wave * 1024;
        if (mode == 1) {
            for (; kt + 1 < KT; ++kt) {
                MOE_THIN_ARGS(kt)
                gemm_tile_asm_thin<OB1, OB2, OB3>(c, x, ra[1] + so, rb[1] + sbo, ra[2] + so, rb[2] + sbo,
                                                  ra[3] + so, rb[3] + sbo, ra[0] + no, rb[0] + nbo, vo, At + koff,
                                                  bbase[0] + koff, bbase[1] + koff, bbase[2] + koff,
                                                  bbase[3] + koff, ldsA, ldsB);
            }
        } else {
            for (; kt + 1 < KT; ++kt) {
                MOE_THIN_ARGS(kt)
                (void)so;
                (void)no;
                (void)sbo;
                (void)nbo;
                gemm_tile_asm_loads_only_thin(c, x, vo, At + koff, bbase[0] + koff, bbase[1] + koff,
                                              bbase[2] + koff, bbase[3] + koff, ldsA, ldsB);
            }
        }
#undef MOE_THIN_ARGS
    } else {
#define MOE_TILE_ARGS(kt_)                                                                               \
    const uint32_t so = ((kt_) & 1) * STAGE, no = STAGE - so;                                            \
    const uint32_t sbo = sb * STAGE, nbo = (sb == 2 ? 0 : sb + 1) * STAGE;                               \
    const uint32_t lbo = (sb == 0 ? 2 : sb - 1) * STAGE;   /* stage of weight tile kt + 2 */          \
    const int64_t koff = (int64_t)((kt_) + 2) * BK;                                                      \
    const int64_t kbo = koff;
    if (mode == 2) {
        for (; kt + 2 < KT; ++kt) {
            MOE_TILE_ARGS(kt)
            gemm_tile_asm<OB1, OB2, OB3>(c, x, ra[1] + so, rb[1] + sbo, ra[2] + so, rb[2] + sbo, ra[3] + so,
                                         rb[3] + sbo, ra[0] + no, rb[0] + nbo, vo, At + koff, bbase[0] + kbo,
                                         bbase[1] + kbo, bbase[2] + kbo, bbase[3] + kbo,
                                         sA_addr + so + wave * 1024, sB_addr + lbo + wave * 1024);
            sb = sb == 2 ? 0 : sb + 1;
        }
    } else if (mode == 1) {
        for (; kt + 2 < KT; ++kt) {
            MOE_TILE_ARGS(kt)
            gemm_tile_asm_half<OB1, OB2, OB3>(c, x, ra[1] + so, rb[1] + sbo, ra[2] + so, rb[2] + sbo, ra[3] + so,
                                              rb[3] + sbo, ra[0] + no, rb[0] + nbo, vo, At + koff, bbase[0] + kbo,
                                              bbase[1] + kbo, bbase[2] + kbo, bbase[3] + kbo,
                                              sA_addr + so + wave * 1024, sB_addr + lbo + wave * 1024);
            sb = sb == 2 ? 0 : sb + 1;
        }
    } else {
        for (; kt + 2 < KT; ++kt) {
            MOE_TILE_ARGS(kt)
            (void)no;
            (void)nbo;
            gemm_tile_asm_loads_only(c, x, vo, At + koff, bbase[0] + kbo, bbase[1] + kbo, bbase[2] + kbo,
                                     bbase[3] + kbo, sA_addr + so + wave * 1024, sB_addr + lbo + wave * 1024);
            sb = sb == 2 ? 0 : sb + 1;
        }
    }
#undef MOE_TILE_ARGS
    }
    // the last (up to) two tiles: nothing left to load
    for (; kt < KT; ++kt) {
        const int ao = aoff_of(kt), bo = boff_of(kt);
        bf16x8_t y[6];
        read_sub(ao, bo, 1, y);
        mma(x);
        read_sub(ao, bo, 2, x);
        mma(y);
        read_sub(ao, bo, 3, y);
        mma(x);
        if (kt + 1 < KT) {
            wait_tiles<8>(0);
            lds_barrier_reads_done();
            read_sub(aoff_of(kt + 1), boff_of(kt + 1), 0, x);
        }
        mma(y);
    }
    // thin tiles may still have loads past the last tile in flight: they must land
    // before the workgroup's LDS is released
    if (thin) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Epilogue: the lane holds output row (.. + lrow) of accumulator q and, in
    // register group g, columns 8 g + 4 lhalf + 0..3 of its 32-column fragment.
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int i = q % 2, f = q / 2;
        const int o = NOPS == 2 ? f / NTW : 0, j = NOPS == 2 ? f % NTW : f;
        if (SWIGLU && o == 1) continue;
        if (thin && i == 1) continue;   // rows of the next wave's half
        const int64_t row = tc.row_start + arow + i * 32 + lrow;
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int col = n0 + wn * WN + j * 32 + 8 * g + 4 * lhalf;
            if (col >= N) continue;   // N % 8 == 0: a group of 4 is wholly in or out
            if (swiglu_part) {
                const int v = 4 * g, qu = q + 2 * NTW;
                float* Gp = Cpart + (int64_t)split * part_stride + row * N + col;
                float* Up = Cpart + (int64_t)(S + split) * part_stride + row * N + col;
                *reinterpret_cast<float4*>(Gp) = make_float4(c[q][v], c[q][v + 1], c[q][v + 2], c[q][v + 3]);
                *reinterpret_cast<float4*>(Up) = make_float4(c[qu][v], c[qu][v + 1], c[qu][v + 2], c[qu][v + 3]);
            } else if (SWIGLU) {
                uint32_t p[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int v = 4 * g + 2 * e;
                    const float h0 = silu_f32(c[q][v]) * c[q + 2 * NTW][v];
                    const float h1 = silu_f32(c[q][v + 1]) * c[q + 2 * NTW][v + 1];
                    p[e] = pack_bf16x2(h0, h1);
                }
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + row * N + col) = make_uint2(p[0], p[1]);
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(C) + row * N + col) =
                    make_float4(c[q][4 * g], c[q][4 * g + 1], c[q][4 * g + 2], c[q][4 * g + 3]);
            }
        }
    }
}

// H[r] += P_0[r] + P_1[r] + ... (P_p = H1 + p stride, added in that order) for the
// rows r < offsets[G] (or nrows without offsets): folds the K-split partials into
// the first where the caller wants H itself.
__global__ __launch_bounds__(256) void add_partial_kernel(float* __restrict__ H, const float* __restrict__ H1, int np,
                                                          int64_t stride, const int32_t* __restrict__ offsets, int G,
                                                          int64_t nrows, int N) {
    const int64_t rows = offsets ? offsets[G] : nrows;
    const int64_t n4 = rows * (N / 4);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        float4 a = reinterpret_cast<float4*>(H)[i];
        for (int p = 0; p < np; ++p) {
            const float4 b = reinterpret_cast<const float4*>(H1 + (int64_t)p * stride)[i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        reinterpret_cast<float4*>(H)[i] = a;
    }
}

// h = SiLU(g) * u rounded to bf16, g and u the sums over the S K-split partials
// (gate partial s at part + s stride, up at part + (S + s) stride, added in split
// order), for the rows r < offsets[G] (or nrows); N % 8 == 0.
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(const float* __restrict__ part, int S, int64_t stride,
                                                            const int32_t* __restrict__ offsets, int G,
                                                            int64_t nrows, int N, uint16_t* __restrict__ h) {
    const int64_t rows = offsets ? offsets[G] : nrows;
    const int64_t n4 = rows * (N / 4);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        float4 g = reinterpret_cast<const float4*>(part)[i];
        float4 u = reinterpret_cast<const float4*>(part + (int64_t)S * stride)[i];
        for (int s = 1; s < S; ++s) {
            const float4 gs = reinterpret_cast<const float4*>(part + (int64_t)s * stride)[i];
            const float4 us = reinterpret_cast<const float4*>(part + (int64_t)(S + s) * stride)[i];
            g.x += gs.x;
            g.y += gs.y;
            g.z += gs.z;
            g.w += gs.w;
            u.x += us.x;
            u.y += us.y;
            u.z += us.z;
            u.w += us.w;
        }
        const uint32_t p0 = pack_bf16x2(silu_f32(g.x) * u.x, silu_f32(g.y) * u.y);
        const uint32_t p1 = pack_bf16x2(silu_f32(g.z) * u.z, silu_f32(g.w) * u.w);
        reinterpret_cast<uint2*>(h)[i] = make_uint2(p0, p1);
    }
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM (plain FMA)
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Grouped GEMV for a handful of rows per group (decode batches)
// ---------------------------------------------------------------------------
//
// With at most MOE_GEMV_ROWS rows in every group the expert GEMMs are weight
// streams (a few flops per weight byte): no LDS staging, no MFMA.  Each wave owns
// 4 weight rows over the whole K, 8 when the groups have one row (SwiGLU: the
// gate and up rows of half as many output columns); per step a lane loads 16 bytes (8 bf16)
// of each weight row and of each of the group's activation rows at K offset
// 8 lane + 512 step and accumulates exact bf16 products in fp32; the 64 lanes'
// partial sums are then added by a butterfly.  Small register and no LDS
// footprint, so many waves per CU keep enough weight loads in flight.
// Workgroup b: the (b / nchunk)-th group with rows (the active groups, found
// with a ballot over offsets), output columns from (b % nchunk) * 4 waves.
// Weight rows per wave for an instance with at most `rmax` activation rows: with
// one row the accumulators are few, so 8 rows (twice the loads per step) fit.
__host__ __device__ constexpr int gemv_rows_per_wave(int rmax) { return rmax == 1 ? 8 : 4; }
// 8 bf16 products added to acc in fp32.  DOT2: four v_dot2c_f32_bf16 on the
// packed operands (a pair of exact products per instruction: a third of the
// VALU work, which matters from 4 activation rows on); otherwise eight FMAs on
// the upcast values (measured faster with one or two rows).
template <bool DOT2>
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (DOT2) {
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, av[i]),
                                                  __builtin_bit_cast(bf16x2_t, bv[i]), acc, false);
        } else {
            acc = fmaf(__uint_as_float(av[i] << 16), __uint_as_float(bv[i] << 16), acc);
            acc = fmaf(__uint_as_float(av[i] & 0xffff0000u), __uint_as_float(bv[i] & 0xffff0000u), acc);
        }
    }
    return acc;
}

template <bool SWIGLU, int RMAX>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ B0,
                                                        const uint16_t* __restrict__ B1, void* __restrict__ Cout,
                                                        const int32_t* __restrict__ offsets, int G, int64_t nrows,
                                                        int N, int K, int nchunk,
                                                        const int32_t* __restrict__ gather) {
    constexpr int UNROLL = RMAX <= 4 ? 2 : 1;   // K steps in flight per wave
    constexpr int RW = gemv_rows_per_wave(RMAX);
    constexpr int COLS_W = SWIGLU ? RW / 2 : RW;   // output columns per wave
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int a = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    int g = 0;
    int64_t r0 = 0, r1 = nrows;
    if (offsets) {
        // the a-th group with rows (uniform loop: a, seen and the ballots are)
        g = -1;
        int seen = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int gg = g0 + lane;
            const bool ne = gg < G && offsets[gg + 1] > offsets[gg];
            unsigned long long m = __ballot(ne);
            const int cnt = __popcll(m);
            if (a < seen + cnt) {
                for (int i = a - seen; i > 0; --i) m &= m - 1;
                g = g0 + __builtin_ctzll(m);
                break;
            }
            seen += cnt;
        }
        if (g < 0) return;
        r0 = offsets[g];
        r1 = offsets[g + 1];
    } else if (a > 0) {
        return;
    }
    const int R = (int)min<int64_t>(r1 - r0, RMAX);
    const int c0 = (chunk * 4 + wave) * COLS_W;
    if (R <= 0 || c0 >= N) return;
    if (r1 - r0 > RMAX) {
        // more rows than the bound the host sized RMAX by (offsets a dispatch would
        // not build): the rows past it are not computed, so they are set to NaN
        // rather than left holding stale values
        for (int64_t i = lane; i < (r1 - r0 - RMAX) * COLS_W; i += 64) {
            const int64_t row = r0 + RMAX + i / COLS_W;
            const int col = c0 + (int)(i % COLS_W);
            if (col >= N) continue;
            if (SWIGLU) static_cast<uint16_t*>(Cout)[row * N + col] = 0x7fc0;
            else static_cast<float*>(Cout)[row * N + col] = __int_as_float(0x7fc00000);
        }
    }
    const int64_t wstride = (int64_t)N * K;
    const uint16_t* wrow[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        const int col = c0 + (SWIGLU ? q % COLS_W : q);
        const uint16_t* base = (SWIGLU && q >= COLS_W ? B1 : B0) + (int64_t)g * wstride;
        wrow[q] = base + (int64_t)(col < N ? col : 0) * K;   // columns past N read column 0, never stored
    }
    const uint16_t* xrow[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        const int64_t row = r0 + (r < R ? r : 0);
        xrow[r] = A + (gather ? (int64_t)gather[row] : row) * K;
    }
    float acc[RMAX][RW];
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
#pragma unroll
        for (int q = 0; q < RW; ++q) acc[r][q] = 0.f;
#pragma unroll UNROLL
    for (int k = lane * 8; k < K; k += 512) {
        uint4 w[RW];
#pragma unroll
        for (int q = 0; q < RW; ++q) w[q] = gload16(wrow[q] + k);
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            if (r < R) {
                const uint4 xv = gload16(xrow[r] + k);
#pragma unroll
                for (int q = 0; q < RW; ++q) acc[r][q] = dot8_bf16<(RMAX >= 4)>(xv, w[q], acc[r][q]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        if (r < R) {
#pragma unroll
            for (int q = 0; q < RW; ++q) acc[r][q] = wave_sum(acc[r][q]);
        }
    }
    if (lane != 0) return;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        if (r >= R) break;
        const int64_t row = r0 + r;
        if (SWIGLU) {
#pragma unroll
            for (int c = 0; c < COLS_W; ++c) {
                if (c0 + c < N)
                    static_cast<uint16_t*>(Cout)[row * N + c0 + c] =
                        (uint16_t)f32_to_bf16_bits(silu_f32(acc[r][c]) * acc[r][c + COLS_W]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < RW; ++q)
                if (c0 + q < N) static_cast<float*>(Cout)[row * N + c0 + q] = acc[r][q];
        }
    }
}

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

// The scheduled kernel's conditions: whole K tiles of 64, 4-column output groups,
// 32-bit load offsets within a 256-row tile.
// Width of the column super-tiles an XCD walks through (see tile_coords).  With
// groups of at most one row tile on average, a wide super-tile lets the
// workgroups an XCD runs together reuse the same activation rows across many
// weight tiles; otherwise 4 keeps both operands' tiles shared.
int super_width(int64_t max_rows, int G, int NT) {
    return (G > 1 && max_rows <= (int64_t)G * 256) ? std::min(NT, 16) : NSUPER;
}

bool asm_path_ok(int N, int K) { return K % 64 == 0 && N % 8 == 0 && (int64_t)K * 512 < ((int64_t)1 << 32); }

hipError_t prep_tiles(const int32_t* offsets, int G, int BM, void* ws, hipStream_t st) {
    if (!offsets) return hipSuccess;
    hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, st, offsets, G, BM, static_cast<int32_t*>(ws));
    return hipGetLastError();
}

// Counter set `set` of the balanced schedule (grouped launches only): set 0 for
// GEMM1, set 1 for GEMM2.  Launches whose whole grid fits in one round of
// workgroups (small batches) keep the static schedule: every workgroup starts at
// once, so there is no tail to balance and a claim would only add its latency.
unsigned long long* sched_set(const int32_t* offsets, void* ws, int G, int set) {
    return offsets ? moe_sched_words(static_cast<int32_t*>(ws), G) + set * XCDS : nullptr;
}

unsigned grid_size(const int32_t* offsets, int G, int64_t max_rows, int BM, int N, int BN) {
    const int64_t mt = (max_rows + BM - 1) / BM + (offsets ? G : 0);
    const int64_t nt = (N + BN - 1) / BN;
    return (unsigned)(mt * nt);
}

}  // namespace

namespace moe_kernels {

// tile prefix (G + 1 int32, padded to 8 bytes) and the balanced schedule's counters
size_t gemm_ws_bytes(int G) {
    return ((size_t)((G + 2) & ~1) * sizeof(int32_t) + MOE_SCHED_WORDS * sizeof(unsigned long long) + 255) &
           ~(size_t)255;
}

int gemm_tile_rows(int dtype) { return dtype == MOE_BF16 ? BF16_BM : F32_BM; }

// K splits for a grouped GEMM with few row tiles (small batches: every active
// group then holds about one row tile, and the tiles stream weights from HBM):
// as many copies of the tile grid as still fit in one round on the CUs — a round
// of fewer, longer workgroups streamed faster than several rounds of short ones —
// at most 16 and at least 4 K tiles per split.  Depends on the shape only
// (workspace sizes follow from it).
int64_t est_tiles(int64_t max_rows, int G, int N, int BN) {
    const int64_t groups = std::max<int64_t>(std::min<int64_t>(G, max_rows), (max_rows + BF16_BM - 1) / BF16_BM);
    return std::max<int64_t>(1, groups * ((N + BN - 1) / BN));
}

int small_splits(int64_t max_rows, int G, int N, int BN, int K) {
    const int S = (int)std::min<int64_t>(16, MOE_GEMM_CUS / est_tiles(max_rows, G, N, BN));
    return std::max(1, std::min(S, (K / 64) / 4));
}

// whole grid (tiles x splits) expected to fit in one round on the CUs
int one_round(int64_t max_rows, int G, int N, int BN, int S) {
    return est_tiles(max_rows, G, N, BN) * S <= MOE_GEMM_CUS ? 1 : 0;
}

bool gemv_path(int dtype, int64_t group_rows) { return dtype == MOE_BF16 && group_rows <= MOE_GEMV_ROWS; }

int gemm1_splits(int dtype, int64_t max_rows, int G, int N, int K, int64_t group_rows) {
    if (dtype != MOE_BF16 || !asm_path_ok(N, K) || gemv_path(dtype, group_rows)) return 1;
    return small_splits(max_rows, G, N, BF16_BN1, K);
}

size_t gemm1_part_bytes(int dtype, int64_t max_rows, int G, int N, int K, int64_t group_rows) {
    const int S = gemm1_splits(dtype, max_rows, G, N, K, group_rows);
    return S > 1 ? (size_t)2 * S * max_rows * N * sizeof(float) : 0;
}

bool gemm1_gather_ok(int dtype, int N, int K, int64_t a_rows) {
    return dtype == MOE_BF16 && asm_path_ok(N, K) && a_rows * K * 2 < ((int64_t)1 << 32);
}

// Grouped GEMV launch: one workgroup per (group with rows, chunk of 4 waves'
// output columns); at most min(G, max_rows) groups have rows.
template <bool SWIGLU, int RMAX>
hipError_t launch_gemv_rows(const void* A, const int32_t* offsets, int G, int64_t max_rows, const void* B0,
                            const void* B1, void* C, int N, int K, const int32_t* gather, hipStream_t st) {
    constexpr int RW = gemv_rows_per_wave(RMAX);
    const int cols_wg = 4 * (SWIGLU ? RW / 2 : RW);   // 4 waves per workgroup
    const int nchunk = (N + cols_wg - 1) / cols_wg;
    const int64_t groups = offsets ? std::min<int64_t>(G, max_rows) : 1;
    hipLaunchKernelGGL((gemv_bf16_kernel<SWIGLU, RMAX>), dim3((unsigned)(groups * nchunk)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(B0),
                       static_cast<const uint16_t*>(B1), C, offsets, G, max_rows, N, K, nchunk, gather);
    return hipGetLastError();
}

// the row bound picks the instance (registers for that many activation rows)
template <bool SWIGLU>
hipError_t launch_gemv(const void* A, const int32_t* offsets, int G, int64_t max_rows, int64_t group_rows,
                       const void* B0, const void* B1, void* C, int N, int K, const int32_t* gather,
                       hipStream_t st) {
    if (max_rows <= 0 || group_rows <= 0 || N <= 0) return hipSuccess;
    if (group_rows <= 1) return launch_gemv_rows<SWIGLU, 1>(A, offsets, G, max_rows, B0, B1, C, N, K, gather, st);
    if (group_rows <= 2) return launch_gemv_rows<SWIGLU, 2>(A, offsets, G, max_rows, B0, B1, C, N, K, gather, st);
    if (group_rows <= 4) return launch_gemv_rows<SWIGLU, 4>(A, offsets, G, max_rows, B0, B1, C, N, K, gather, st);
    return launch_gemv_rows<SWIGLU, (int)MOE_GEMV_ROWS>(A, offsets, G, max_rows, B0, B1, C, N, K, gather, st);
}

hipError_t launch_gemm1(int dtype, const void* A, const int32_t* offsets, int G, int64_t max_rows, const void* w_gate,
                        const void* w_up, void* h, int N, int K, void* ws, hipStream_t st, bool prefix_ready,
                        float* part, const int32_t* gather, int64_t group_rows) {
    if (gemv_path(dtype, group_rows))
        return launch_gemv<true>(A, offsets, G, max_rows, group_rows, w_gate, w_up, h, N, K, gather, st);
    const int BM = dtype == MOE_BF16 ? BF16_BM : F32_BM;
    const int BN = dtype == MOE_BF16 ? BF16_BN1 : F32_BN;
    hipError_t e = prefix_ready ? hipSuccess : prep_tiles(offsets, G, BM, ws, st);
    if (e != hipSuccess) return e;
    unsigned grid = grid_size(offsets, G, max_rows, BM, N, BN);
    if (grid == 0) return hipSuccess;
    const int32_t* tp = static_cast<const int32_t*>(ws);
    const int S = part ? gemm1_splits(dtype, max_rows, G, N, K, group_rows) : 1;
    if (dtype == MOE_BF16 && asm_path_ok(N, K) && S > 1) {
        // fp32 gate / up partials per K split, then SiLU(g) * u from their sums
        grid = (grid + XCDS - 1) / XCDS * XCDS * S;
        const int64_t stride = max_rows * N;
        hipLaunchKernelGGL((gemm_bf16_asm_kernel<BF16_BN1, true, true>), dim3(grid), dim3(512), 0, st,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(w_gate),
                           static_cast<const uint16_t*>(w_up), h, part, stride, offsets, tp, G, max_rows, N, K, S,
                           NSUPER, one_round(max_rows, G, N, BF16_BN1, S), gather, (unsigned long long*)nullptr);
        const int64_t n4 = max_rows * (N / 4);
        hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((unsigned)std::min<int64_t>((n4 + 255) / 256, 8192)),
                           dim3(256), 0, st, part, S, stride, offsets, G, max_rows, N, static_cast<uint16_t*>(h));
    } else if (dtype == MOE_BF16 && asm_path_ok(N, K))
        hipLaunchKernelGGL((gemm_bf16_asm_kernel<BF16_BN1, true>), dim3(grid), dim3(512), 0, st,
                           static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(w_gate),
                           static_cast<const uint16_t*>(w_up), h, nullptr, (int64_t)0, offsets, tp, G, max_rows, N, K, 1,
                           NSUPER, one_round(max_rows, G, N, BF16_BN1, 1), gather,
                           one_round(max_rows, G, N, BF16_BN1, 1) ? nullptr : sched_set(offsets, ws, G, 0));
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

int gemm2_splits(int dtype, int64_t max_rows, int G, int N, int K, int64_t group_rows) {
    if (dtype != MOE_BF16 || !asm_path_ok(N, K) || gemv_path(dtype, group_rows)) return 1;
    const int s_small = small_splits(max_rows, G, N, BF16_BN2, K);
    if (s_small > 1) return s_small;
    if (K % 128 != 0 || K < 2048) return 1;
    // expected row tiles: full tiles plus about half a partial tile per group
    const int64_t mt = (max_rows + BF16_BM - 1) / BF16_BM + (G + 1) / 2;
    const int64_t tiles = mt * ((N + BF16_BN2 - 1) / BF16_BN2);
    auto fill = [](int64_t t) {   // fraction of the CU slots the workgroups' rounds use
        const int64_t rounds = (t + MOE_GEMM_CUS - 1) / MOE_GEMM_CUS;
        return rounds ? (double)t / (double)(rounds * MOE_GEMM_CUS) : 1.0;
    };
    return fill(2 * tiles) > 1.05 * fill(tiles) ? 2 : 1;
}

hipError_t launch_gemm2(int dtype, const void* h, const int32_t* offsets, int G, int64_t max_rows,
                        const void* w_down, float* H, float* H1, int N, int K, void* ws, hipStream_t st,
                        bool prefix_ready, int64_t group_rows) {
    if (gemv_path(dtype, group_rows))
        return launch_gemv<false>(h, offsets, G, max_rows, group_rows, w_down, nullptr, H, N, K, nullptr, st);
    const int BM = dtype == MOE_BF16 ? BF16_BM : F32_BM;
    const int BN = dtype == MOE_BF16 ? BF16_BN2 : F32_BN;
    hipError_t e = prefix_ready ? hipSuccess : prep_tiles(offsets, G, BM, ws, st);
    if (e != hipSuccess) return e;
    unsigned grid = grid_size(offsets, G, max_rows, BM, N, BN);
    if (grid == 0) return hipSuccess;
    const int32_t* tp = static_cast<const int32_t*>(ws);
    const int S = H1 ? gemm2_splits(dtype, max_rows, G, N, K, group_rows) : 1;
    if (dtype == MOE_BF16 && asm_path_ok(N, K)) {
        if (S > 1) grid = (grid + XCDS - 1) / XCDS * XCDS * S;
        hipLaunchKernelGGL((gemm_bf16_asm_kernel<BF16_BN2, false>), dim3(grid), dim3(512), 0, st,
                           static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), nullptr, H, H1,
                           max_rows * N, offsets, tp, G, max_rows, N, K, S,
                           super_width(max_rows, G, (N + BN - 1) / BN), one_round(max_rows, G, N, BF16_BN2, S),
                           (const int32_t*)nullptr,
                           one_round(max_rows, G, N, BF16_BN2, S) ? nullptr : sched_set(offsets, ws, G, 1));
    } else if (dtype == MOE_BF16) {
        hipLaunchKernelGGL((gemm_bf16_kernel<BF16_BM, BF16_BN2, false>), dim3(grid), dim3(256), 0, st,
                           static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_down), nullptr, H,
                           offsets, tp, G, max_rows, N, K);
    } else {
        hipLaunchKernelGGL((gemm_f32_kernel<false>), dim3(grid), dim3(256), 0, st, static_cast<const float*>(h),
                           static_cast<const float*>(w_down), nullptr, H, offsets, tp, G, max_rows, N, K);
    }
    return hipGetLastError();
}

int scores_splits(int64_t T, int N, int K) {
    if (!asm_path_ok(N, K)) return 1;
    const int64_t tiles = ((T + BF16_BM - 1) / BF16_BM) * ((N + BF16_BN2 - 1) / BF16_BN2);
    const int KT = K / 64;
    int S = (int)std::min<int64_t>(16, std::max<int64_t>(1, MOE_GEMM_CUS / std::max<int64_t>(tiles, 1)));
    return std::max(1, std::min(S, KT / 4));   // at least 4 K tiles per split
}

hipError_t launch_scores_gemm(const void* x, const void* w, int64_t T, int N, int K, float* part, hipStream_t st) {
    const unsigned tiles = grid_size(nullptr, 1, T, BF16_BM, N, BF16_BN2);
    if (tiles == 0) return hipSuccess;
    const int S = scores_splits(T, N, K);
    if (asm_path_ok(N, K)) {
        const unsigned grid = (tiles + XCDS - 1) / XCDS * XCDS * S;
        hipLaunchKernelGGL((gemm_bf16_asm_kernel<BF16_BN2, false>), dim3(grid), dim3(512), 0, st,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), nullptr, part,
                           part + T * N, T * N, nullptr, nullptr, 1, T, N, K, S, NSUPER, 0, (const int32_t*)nullptr,
                           (unsigned long long*)nullptr);
    } else {
        hipLaunchKernelGGL((gemm_bf16_kernel<BF16_BM, BF16_BN2, false>), dim3(tiles), dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), nullptr, part, nullptr,
                           nullptr, 1, T, N, K);
    }
    return hipGetLastError();
}

hipError_t launch_add_partial(float* H, const float* H1, int np, const int32_t* offsets, int G, int64_t max_rows,
                              int N, hipStream_t st) {
    const int64_t n4 = max_rows * (N / 4);
    if (n4 == 0 || np == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(add_partial_kernel, dim3(grid), dim3(256), 0, st, H, H1, np, max_rows * N, offsets, G,
                       max_rows, N);
    return hipGetLastError();
}

}  // namespace moe_kernels
