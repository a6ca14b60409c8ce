/*
 * ssm_bwd.h -- C ABI of the backward pass of the selective scan (gfx950).
 *
 * The page "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"
 * ("Hardware-aware state expansion") describes the fused kernel's backward
 * pass: the intermediate states are recomputed on chip rather than stored
 * in and read back from HBM.  ssm_scan_bwd returns the gradients of
 *     l = sum(dy * y) + sum(dhL * hL)
 * with respect to every input of ssm_scan_fwd (see ssm.h for the forward map
 * and layouts), for the Delta * B form of B-bar or, with SSM_FLAG_ZOH_B, the
 * exact zero-order-hold form.  flags may also hold SSM_FLAG_CHECKPOINTS:
 * `workspace` then already holds the checkpoints that ssm_scan_fwd wrote
 * with that flag for the same x, dt, dt_bias, A, Bm, h0 and form of B-bar,
 * and the recomputation pass is skipped.
 *
 * Per (b, d), with u_t = dt_t + dt_bias, Delta_t = softplus(u_t),
 * A-bar_t = exp(Delta_t A), s_t = C_t . h_t + Dskip x_t, ds_t = dy_t silu(z_t):
 *     lambda_t = ds_t C_t + A-bar_{t+1} lambda_{t+1},  lambda_{L-1} = ds C + dhL
 *     dx_t = Dskip ds_t + sum_n lambda_t Delta_t B_t
 *     ddt_t = sigmoid(u_t) sum_n lambda_t (A A-bar_t h_{t-1} + B_t x_t)
 *     dz_t = dy_t s_t silu'(z_t)
 *     dBm[b,n,t] = sum_d lambda_t Delta_t x_t,   dCm[b,n,t] = sum_d ds_t h_t
 *     dA[d,n] = sum_{b,t} lambda_t Delta_t A-bar_t h_{t-1}
 *     dDskip[d] = sum_{b,t} ds_t x_t,  ddt_bias[d] = sum_{b,t} ddt_t
 *     dh0 = A-bar_0 lambda_0
 * With SSM_FLAG_ZOH_B the input term Delta_t B_t x_t becomes g_t B_t x_t,
 * g = (exp(Delta A) - 1) / A (Delta at A = 0; "Method" section): Delta_t is
 * replaced by g_t in dx and dBm, the B_t x_t term of ddt gains the factor
 * dg/dDelta = A-bar_t, and dA gains sum_{b,t} lambda_t B_t x_t dg/dA with
 * dg/dA = Delta^2 psi(Delta A), psi(u) = (u e^u - (e^u - 1)) / u^2.
 *
 * Conventions are those of ssm.h (caller-owned device pointers, densely
 * packed, nothing allocated; argument errors return before any launch and
 * write nothing; SSM_ERR_HIP on a failed launch; asynchronous on `stream`).
 * The sums over channels and over batch and time are accumulated with fp32
 * atomic adds, so their rounding (not their value) may differ between runs.
 */
#ifndef SSM_BWD_H
#define SSM_BWD_H

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Device workspace ssm_scan_bwd needs: the state entering every 64-step
 * chunk (batch * dim * ceil(seqlen / 64) * dstate fp32 values, first) and 8
 * partial copies of dBm and dCm (8 * 2 * batch * dstate * seqlen fp32), or,
 * if larger, the forward's sequence-split workspace
 * (ssm_scan_fwd_workspace_bytes), which a forward with SSM_FLAG_CHECKPOINTS
 * keeps after the checkpoints; for a split shape, as many bytes again as the
 * forward's split workspace follow (the backward's own adjoint planes).  A function of the sizes
 * only; sizes ssm_scan_bwd would refuse (batch, dim or seqlen below 1,
 * batch above 65535, seqlen above 2^28 - 4096, dstate not in {1, 2, 4, 8,
 * 16}) give 0. */
size_t ssm_scan_bwd_workspace_bytes(int batch, int dim, int seqlen, int dstate);

/*
 * Inputs: the forward inputs exactly as given to ssm_scan_fwd, plus
 *   dy       [batch][dim][seqlen]  grad_dtype  gradient of y
 *   dhL      [batch][dim][dstate]  fp32 gradient of the final state, or NULL (zero)
 * Outputs (all overwritten; none may overlap an input, another output or
 * the workspace):
 *   dx, ddt  [batch][dim][seqlen]  grad_dtype (ddt: gradient of the raw dt)
 *   dz       [batch][dim][seqlen]  grad_dtype; required when z is given,
 *            ignored (may be NULL) otherwise
 *   dBm, dCm [batch][dstate][seqlen] fp32
 *   dA       [dim][dstate] fp32
 *   dDskip, ddt_bias [dim] fp32, or NULL (not computed)
 *   dh0      [batch][dim][dstate] fp32, or NULL (not returned)
 *   workspace, workspace_bytes: at least ssm_scan_bwd_workspace_bytes(...)
 * Supported sizes: as ssm_scan_fwd.
 */
ssm_status_t ssm_scan_bwd(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype,
                          unsigned flags, const void *x, const void *dt, const float *dt_bias,
                          const float *A, const void *Bm, const void *Cm, const float *Dskip,
                          const void *z, const float *h0, ssm_dtype_t grad_dtype,
                          const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                          float *dBm, float *dCm, float *dA, float *dDskip, float *ddt_bias,
                          float *dh0, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Strided layouts for ssm_scan_bwd_strided, in the manner of
 * ssm_scan_layout_t (ssm.h): strides in ELEMENTS of each tensor's own type,
 * time contiguous.  In training, z comes from the same input projection as
 * x, and its gradient dz goes back into that projection's gradient buffer,
 * so both are usually halves of one [batch][2 dim][seqlen] buffer.
 *   seq_row        distance between rows (channels) of x, dt, z, dy, dx,
 *                  ddt and dz, shared by the seven; >= seqlen; 0 means seqlen
 *   seq_batch[7]   distance between batch entries of x, dt, z, dy, dx, ddt,
 *                  dz (in that order); each >= dim * seq_row; 0 means
 *                  dim * seq_row
 *   bc_row, bc_batch[2]  as in ssm_scan_layout_t, for Bm and Cm
 * dBm, dCm and every other argument stay dense.  The limits and errors are
 * those of ssm_scan_layout_t; overlap is checked on each tensor's address
 * range from its first to its last element, so two outputs (dx and dz, say)
 * may not be interleaved halves of one buffer, while dz alone may be written
 * into half of one.
 */
typedef struct {
    long long seq_row;
    long long seq_batch[7];
    long long bc_row;
    long long bc_batch[2];
} ssm_scan_bwd_layout_t;

/*
 * ssm_scan_bwd on strided views: the same arguments, flags and errors, with
 * `layout` (host pointer, read during the call only; NULL means dense).
 */
ssm_status_t ssm_scan_bwd_strided(int batch, int dim, int seqlen, int dstate,
                                  ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, ssm_dtype_t grad_dtype,
                                  const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                                  float *dBm, float *dCm, float *dA, float *dDskip,
                                  float *ddt_bias, float *dh0, void *workspace,
                                  size_t workspace_bytes, const ssm_scan_bwd_layout_t *layout,
                                  void *stream);

/*
 * The backward pass on (batch, L, dim)-ordered tensors, the layout of
 * ssm_scan_fwd_bld (ssm.h): a time step's channels (states) contiguous, time
 * steps apart.  Strides in ELEMENTS of each tensor's own type:
 *   x, dt, z, dy, dx, ddt, dz (index i = 0..6 in that order): element
 *            (b, t, d) at b * batch_stride[i] + t * step[i] + d;
 *            step[i] >= dim (0 means dim), batch_stride[i] >= seqlen * step
 *            (0 means seqlen * step)
 *   Bm, Cm   element (b, t, n) at b * *_batch + t * *_step + n, limits as
 *            in ssm_bld_layout_t (B_step, C_step >= dstate)
 * A negative stride, one below its minimum, a step stride above 2^40 or a
 * tensor spanning 2^56 elements or more is SSM_ERR_BAD_SHAPE.  A NULL
 * layout means all zero (dense).
 */
typedef struct {
    long long step[7];
    long long batch_stride[7];
    long long B_step, C_step, B_batch, C_batch;
} ssm_scan_bwd_bld_layout_t;

/* Device workspace ssm_scan_bwd_bld needs, in bytes: seven
 * [batch][dim][seqlen] and four [batch][dstate][seqlen] planes sized for fp32
 * (each rounded up to 256 bytes), then ssm_scan_bwd_workspace_bytes(...).
 * 0 for sizes it refuses (as ssm_scan_bwd_workspace_bytes, and sizes whose
 * workspace would reach 2^62 bytes, which ssm_scan_bwd_bld refuses with
 * SSM_ERR_BAD_SHAPE). */
size_t ssm_scan_bwd_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate);

/*
 * ssm_scan_bwd on (batch, L, dim)-ordered tensors laid out by `layout` (host
 * pointer, read during the call only).  The same arguments, gradients (up to
 * the rounding of the atomic sums) and errors as ssm_scan_bwd, with:
 *   dBm, dCm  [batch][seqlen][dstate] fp32, dense
 *   workspace, workspace_bytes: at least ssm_scan_bwd_bld_workspace_bytes(...)
 *   flags     SSM_FLAG_ZOH_B only (ssm_scan_fwd_bld writes no checkpoints:
 *             SSM_FLAG_CHECKPOINTS is SSM_ERR_UNSUPPORTED)
 * The call copies x, dt, z, dy, Bm and Cm into [batch][dim][seqlen] (and
 * [batch][dstate][seqlen]) order in the workspace with tiled transposes
 * (exact copies), runs the backward kernels there, and copies dx, ddt, dz,
 * dBm and dCm back.  Overlap is checked on address ranges from the first to
 * the last element.  Supported sizes: as ssm_scan_fwd.
 */
ssm_status_t ssm_scan_bwd_bld(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype,
                              unsigned flags, const void *x, const void *dt, const float *dt_bias,
                              const float *A, const void *Bm, const void *Cm, const float *Dskip,
                              const void *z, const float *h0, ssm_dtype_t grad_dtype,
                              const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                              float *dBm, float *dCm, float *dA, float *dDskip, float *ddt_bias,
                              float *dh0, void *workspace, size_t workspace_bytes,
                              const ssm_scan_bwd_bld_layout_t *layout, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_BWD_H */
