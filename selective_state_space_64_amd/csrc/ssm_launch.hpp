// ssm_launch.hpp -- internal interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ssm {

struct ScanArgs {
    int batch, dim, seqlen, dstate;
    int in_bf16, out_bf16, zoh;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    void *y;
    float *hL;
    float *ck;  // optional checkpoint output (state entering each 64-step chunk)
    // Strides in elements (time stride is 1): rows of x, dt, z, y are `row`
    // apart, rows of Bm, Cm `bc_row` apart; batch entries `*_b` apart.
    long long row, x_b, dt_b, z_b, y_b, bc_row, B_b, C_b;
    // Workspace of the sequence split (scan_fwd_split_bytes), or NULL when
    // the shape is not split.
    float *agg;
    // Checkpoints only (for the backward pass): no readout, no y, no hL.
    int ckpt_only;
};

// Sequence split of the forward scan: segments of seg_len steps (a multiple
// of the aggregate pass's 256-step chunk) scanned by separate workgroups.  A function of the
// shape only, so that the workspace size is known before the call.
struct ScanSplit {
    int nseg, seg_len;
};
ScanSplit scan_fwd_split(int batch, int dim, int seqlen);
// Bytes of the split's workspace: one plane of (dstate + 1) floats per
// (batch, channel) for every segment; 0 when the shape is not split.
size_t scan_fwd_split_bytes(int batch, int dim, int seqlen, int dstate);

struct UpdateArgs {
    int batch, dim, dstate;
    int in_bf16, out_bf16, zoh;
    float *state;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    void *y;
    // batch strides in elements: x, dt, z, y (rows of dim), Bm, Cm (rows of dstate)
    long long x_b, dt_b, z_b, y_b, B_b, C_b;
};

struct ConvArgs {
    int batch, dim, seqlen, width;
    int in_bf16, out_bf16, silu;
    const void *x;
    const float *weight, *bias, *state0;
    void *y;
    float *stateL;
    // element strides of x and y (time contiguous): rows, batch entries
    long long x_row, x_b, y_row, y_b;
};

// The conv on (batch, L, dim)-ordered x and y: element (b, t, d) at
// b * *_b + t * *_t + d (element strides).
struct ConvBldArgs {
    int batch, dim, seqlen, width;
    int in_bf16, out_bf16, silu;
    const void *x;
    const float *weight, *bias, *state0;
    void *y;
    float *stateL;
    long long x_t, x_b, y_t, y_b;
};

struct ConvUpdateArgs {
    int batch, dim, width;
    int in_bf16, out_bf16, silu;
    float *state;
    const void *x;
    const float *weight, *bias;
    void *y;
    long long x_b, y_b;  // batch strides of x and y in elements
};

struct BwdArgs {
    int batch, dim, seqlen, dstate;
    int in_bf16, grad_bf16;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    const void *dy;
    const float *dhL;
    void *dx, *ddt, *dz;
    float *dBm, *dCm, *dA, *dDskip, *ddt_bias, *dh0;
    void *workspace;
    int ckpt_given;  // the workspace already holds the forward's checkpoints
    // Strides in elements (time stride 1): rows of x, dt, z, dy, dx, ddt, dz
    // `row` apart, rows of Bm, Cm `bc_row` apart, batch entries `*_b` apart.
    long long row, x_b, dt_b, z_b, dy_b, dx_b, ddt_b, dz_b, bc_row, B_b, C_b;
    int zoh;  // the exact zero-order-hold form of B-bar
};

// The backward pass on (batch, L, dim)-ordered tensors: element (b, t, c) of
// x, dt, z, dy, dx, ddt, dz (c < dim) and of Bm, Cm (c < dstate) at
// b * *_b + t * *_t + c (element strides, index i of t[] / b[] in the order
// x, dt, z, dy, dx, ddt, dz); dBm, dCm dense [batch][seqlen][dstate].
struct BwdBldArgs {
    int batch, dim, seqlen, dstate;
    int in_bf16, grad_bf16, zoh;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    const void *dy;
    const float *dhL;
    void *dx, *ddt, *dz;
    float *dBm, *dCm, *dA, *dDskip, *ddt_bias, *dh0;
    void *workspace;  // scan_bwd_bld_workspace_bytes
    long long t[7], b[7];
    long long B_t, B_b, C_t, C_b;
};
size_t scan_bwd_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate);
hipError_t launch_scan_bwd_bld(const BwdBldArgs &a, hipStream_t stream);
// Batched transpose of esize-byte elements (2 or 4): src (b, r, c) at
// src + b s_b + r s_r + c to dst (b, c, r) at dst + b d_b + c d_c + r.
hipError_t launch_transpose(int esize, const void *src, long long s_b, long long s_r, void *dst,
                            long long d_b, long long d_c, int batch, int rows, int cols,
                            hipStream_t stream);

// The forward on (batch, L, dim)-ordered tensors (scan_bld.hip): element
// strides of a time step and of a batch entry for each tensor; the channel
// (x, dt, z, y) or state (Bm, Cm) index is contiguous.
struct BldArgs {
    int batch, dim, seqlen, dstate;
    int in_bf16, out_bf16, zoh;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    void *y;
    float *hL;
    long long x_t, x_b, dt_t, dt_b, z_t, z_b, y_t, y_b, B_t, B_b, C_t, C_b;
    float *workspace;  // scan_bld_workspace_bytes
};
// Pieces of the sequence scanned by separate waves (a function of the shape).
struct BldSplit {
    int npieces, piece_len;
};
BldSplit bld_split(int batch, int dim, int seqlen);
// One record of dstate + 1 floats per piece and (batch, channel).
size_t scan_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate);
hipError_t launch_scan_bld(const BldArgs &a, hipStream_t stream);

// The backward pass keeps the state entering every kCkptSteps-step chunk
// (batch * dim * ceil(seqlen / kCkptSteps) * dstate floats at the start of
// its workspace); the forward writes the same layout with checkpoints on.
constexpr int kCkptSteps = 64;

// The forward's sequence split aims at this many workgroups in all (16
// channels each); it also bounds the split's planes: segments x batch x dim
// <= kSplitTargetWgs x 16.
#ifndef SSM_SPLIT_TARGET_WGS
#define SSM_SPLIT_TARGET_WGS 16384
#endif
constexpr long long kSplitTargetWgs = SSM_SPLIT_TARGET_WGS;
inline size_t scan_checkpoint_floats(int batch, int dim, int seqlen, int dstate)
{
    return size_t(batch) * size_t(dim) * ((size_t(seqlen) + kCkptSteps - 1) / kCkptSteps) *
           size_t(dstate);
}

// Device workspace of the backward pass: the checkpoints, then the partial sums.
size_t scan_bwd_workspace_bytes(int batch, int dim, int seqlen, int dstate);

// All return hipSuccess or the launch error; arguments are already validated.
hipError_t launch_scan_fwd(const ScanArgs &a, hipStream_t stream);
hipError_t launch_state_update(const UpdateArgs &a, hipStream_t stream);
hipError_t launch_conv1d_fwd(const ConvArgs &a, hipStream_t stream);
hipError_t launch_conv1d_bld(const ConvBldArgs &a, hipStream_t stream);
hipError_t launch_conv1d_update(const ConvUpdateArgs &a, hipStream_t stream);
hipError_t launch_scan_bwd(const BwdArgs &a, hipStream_t stream);

// Dispatch log: with the environment variable SSM_LOG set to a non-zero
// value when the library is first used, every launch prints one line to
// stderr (entry point, kernel instantiation, split, grid).  Read once.
bool log_enabled();
void log_line(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
template <typename T>
constexpr const char *type_tag()
{
    return sizeof(T) == 2 ? "bf16" : "f32";
}

// Largest batch the kernels' grids support (grid y dimension).
constexpr int kMaxBatch = 65535;
// Largest dim: channel indices are 32-bit ints inside the kernels (workgroup
// index times channels per workgroup, plus the lane's channel).
constexpr int kMaxDim = 1 << 30;
// Longest sequence: the scan addresses the 4 rows of a wave with 32-bit byte
// offsets, (4 L + 2 chunks) * 4 bytes < 2^32.
constexpr int kMaxSeqlen = (1 << 28) - (1 << 12);

}  // namespace ssm
