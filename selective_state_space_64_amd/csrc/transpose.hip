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
// elements of one row.  Row tiles beyond the grid's y extent (65535) are
// walked by a grid-stride loop.
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
        for (int i = ty; i < kTile; i += 256 / kTile) {
            const int r = r0 + i, c = c0 + tx;
            if (r < rows && c < cols) tile[i][tx] = s[(long long)r * s_r + c];
        }
        __syncthreads();
#pragma unroll
        for (int i = ty; i < kTile; i += 256 / kTile) {
            const int c = c0 + i, r = r0 + tx;
            if (r < rows && c < cols) d[(long long)c * d_c + r] = tile[tx][i];
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
    if (esize == 2) {
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
