// transpose.hip -- batched 2-D transposes between (batch, L, dim) and
// [batch][dim][L] order, for gfx950.
//
// The backward pass on (batch, L, dim)-ordered tensors moves its inputs into
// the [batch][dim][L] order of the backward kernels and its per-step
// gradients back (the (B, L, D) order is the one in which the reading guide
// "Mamba: Linear-Time Sequence Modeling with Selective State Spaces",
// "Hardware-aware state expansion", writes the output back).  Elements are
// moved as raw 16- or 32-bit words: no arithmetic, so the copies are exact.
//
// A workgroup of 256 threads moves 64 x 64 tiles through LDS (one padding
// column, so that the column reads of the second half fall in different
// banks): every global read and write of a wave covers 64 consecutive
// elements of one row, or, where every row is 4-element aligned, 4 rows of 64
// elements in 4-element vectors.  Row tiles beyond the grid's y extent
// (65535) are walked by a grid-stride loop.
#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

constexpr int kTile = 64;

// src element (b, r, c) at src + b s_b + r s_r + c; dst element (b, c, r) at
// dst + b d_b + c d_c + r; r < rows, c < cols.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *src, long long s_b, long long s_r,
                                                        T *dst, long long d_b, long long d_c,
                                                        int rows, int cols)
{
    __shared__ T tile[kTile][kTile + 1];
    const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x / kTile;
    const int c0 = int(blockIdx.x) * kTile;
    const T *s = src + (long long)blockIdx.z * s_b;
    T *d = dst + (long long)blockIdx.z * d_b;
    for (int rt = blockIdx.y; (long long)rt * kTile < rows; rt += gridDim.y) {
        const int r0 = rt * kTile;
        __syncthreads();  // the previous tile has been written out
#pragma unroll
        for (int k = 0; k < kTile / 4; ++k) {
            const int i = ty + 4 * k, r = r0 + i, c = c0 + tx;
            if (r < rows && c < cols) tile[i][tx] = s[(long long)r * s_r + c];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kTile / 4; ++k) {
            const int i = ty + 4 * k, c = c0 + i, r = r0 + tx;
            if (r < rows && c < cols) d[(long long)c * d_c + r] = tile[tx][i];
        }
    }
}

// The same move with 4-element vectors on both sides, for calls whose every
// row of src and dst starts on a multiple of 4 elements of a base aligned to
// 4 elements: a thread reads 4 consecutive elements of a src row (8 or 16
// bytes) and writes 4 consecutive elements of a dst row, gathered from 4 rows
// of the tile.
template <typename T>
__global__ __launch_bounds__(256) void transpose4_kernel(const T *src, long long s_b, long long s_r,
                                                         T *dst, long long d_b, long long d_c,
                                                         int rows, int cols)
{
    typedef T v4 __attribute__((ext_vector_type(4)));
    __shared__ T tile[kTile][kTile + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 16 x 16 threads
    const int c0 = int(blockIdx.x) * kTile;
    const T *s = src + (long long)blockIdx.z * s_b;
    T *d = dst + (long long)blockIdx.z * d_b;
    for (int rt = blockIdx.y; (long long)rt * kTile < rows; rt += gridDim.y) {
        const int r0 = rt * kTile;
        __syncthreads();  // the previous tile has been written out
#pragma unroll
        for (int k = 0; k < kTile / 16; ++k) {
            const int i = ty + 16 * k, r = r0 + i, c = c0 + 4 * tx;
            if (r < rows) {
                if (c + 3 < cols) {
                    const v4 w = *reinterpret_cast<const v4 *>(s + (long long)r * s_r + c);
                    tile[i][4 * tx] = w.x; tile[i][4 * tx + 1] = w.y;
                    tile[i][4 * tx + 2] = w.z; tile[i][4 * tx + 3] = w.w;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (c + q < cols) tile[i][4 * tx + q] = s[(long long)r * s_r + c + q];
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kTile / 16; ++k) {
            const int i = ty + 16 * k, c = c0 + i, r = r0 + 4 * tx;
            if (c < cols) {
                if (r + 3 < rows) {
                    const v4 w = {tile[4 * tx][i], tile[4 * tx + 1][i], tile[4 * tx + 2][i],
                                  tile[4 * tx + 3][i]};
                    *reinterpret_cast<v4 *>(d + (long long)c * d_c + r) = w;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (r + q < rows) d[(long long)c * d_c + r + q] = tile[4 * tx + q][i];
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_transpose(int esize, const void *src, long long s_b, long long s_r, void *dst,
                            long long d_b, long long d_c, int batch, int rows, int cols,
                            hipStream_t stream)
{
    const long long rt = (rows + kTile - 1) / kTile, ct = (cols + kTile - 1) / kTile;
    if (ct > 0x7fffffffLL || batch > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid{unsigned(ct), unsigned(rt < 65535 ? rt : 65535), unsigned(batch)};
    const bool vec = (reinterpret_cast<uintptr_t>(src) % (4 * esize)) == 0 &&
                     (reinterpret_cast<uintptr_t>(dst) % (4 * esize)) == 0 && s_b % 4 == 0 &&
                     s_r % 4 == 0 && d_b % 4 == 0 && d_c % 4 == 0;
    if (vec && esize == 2) {
        hipLaunchKernelGGL(transpose4_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(src), s_b, s_r, static_cast<uint16_t *>(dst),
                           d_b, d_c, rows, cols);
    } else if (vec) {
        hipLaunchKernelGGL(transpose4_kernel<uint32_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint32_t *>(src), s_b, s_r, static_cast<uint32_t *>(dst),
                           d_b, d_c, rows, cols);
    } else if (esize == 2) {
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(src), s_b, s_r, static_cast<uint16_t *>(dst),
                           d_b, d_c, rows, cols);
    } else {
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint32_t *>(src), s_b, s_r, static_cast<uint32_t *>(dst),
                           d_b, d_c, rows, cols);
    }
    return hipGetLastError();
}

}  // namespace ssm
