// Weight repacking: batched transpose, dst[b][j][i] = src[b][i][j].
//
// The pages write the layer as x W with weights stored in-features x
// out-features (router W_r [d,E], gate / up [E,d,m], down [E,m,d]; "LLM from
// scratch" ch. 36 §36.1, and §36.8 on libraries that store the transpose).  The
// kernels here read every weight row along the reduction dimension (16-byte
// MFMA operand loads along K), so they take out x in; this pass converts a
// weight set once, outside the forward.  Pure data movement: the packed values
// are the source's bits.
//
// One 256-thread workgroup per 64 x 64 tile of one matrix: the tile is read row
// by row (consecutive lanes on consecutive columns), kept in LDS with one
// element of padding per row, and written out column by column.
#include "common.h"

namespace {

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows,
                                                        int64_t cols) {
    __shared__ T tile[64][65];
    const int64_t mat = (int64_t)blockIdx.z * rows * cols;
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = src[mat + r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;   // element (r, c) of the source
        if (c < cols && r < rows) dst[mat + c * rows + r] = tile[tx][i];
    }
}

}  // namespace

namespace moe_kernels {

hipError_t launch_transpose(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols, int elem_bytes,
                            hipStream_t st) {
    if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)batch);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(src),
                           static_cast<uint16_t*>(dst), rows, cols);
    else
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, st, static_cast<const uint32_t*>(src),
                           static_cast<uint32_t*>(dst), rows, cols);
    return hipGetLastError();
}

}  // namespace moe_kernels
