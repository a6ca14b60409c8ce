/*
 * ssm_conv.h -- C ABI of the causal depthwise 1-D convolution that feeds the
 * selective scan, and of its single-token decode step (gfx950).
 *
 * The Mamba block applies a short 1-D convolution over the sequence before
 * the selective SSM (glossary entry "Mamba Block" of the page "Mamba:
 * Linear-Time Sequence Modeling with Selective State Spaces"; the basic-model
 * example of the page "Mamba选择性状态空间机制：效率提升10倍的核心突破"
 * uses d_conv = 4).  The inference cache keeps the convolutional state beside
 * the SSM state ("everything-about-mamba-paper", blogofoto.com), and the fast
 * path pairs the scan kernels with a causal conv1d kernel
 * ("details-fiction-and-mamba-paper", dbblog.net).
 *
 * The pages give no formula for the convolution; this library computes, per
 * (batch b, channel d), with e = (state0[b][d][0..W-2], x[b][d][0..L-1]):
 *     y[b][d][t]        = act(bias[d] + sum_{k<W} weight[d][k] * e[t + k])
 *     stateL[b][d][k]   = e[L + k]                    (k < W-1)
 * i.e. a depthwise cross-correlation whose last tap weight[d][W-1] meets the
 * current input, left-padded by the conv state (oldest first) or zeros;
 * act = silu (z * sigmoid(z)) when SSM_CONV_SILU is set, else the identity.
 *
 * Conventions are those of ssm.h: caller-owned, densely packed, row-major
 * device pointers; nothing is allocated or retained; argument errors return a
 * status before anything is enqueued (nothing is written); a failed launch
 * returns SSM_ERR_HIP; calls are asynchronous on `stream` (NULL = default).
 * Every pointer must be aligned to its element size.
 */
#ifndef SSM_CONV_H
#define SSM_CONV_H

#include "ssm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* flags bit 0: apply silu after the bias.  Other bits must be zero
 * (SSM_ERR_UNSUPPORTED). */
#define SSM_CONV_SILU 0x1u

/*
 * Causal conv over whole sequences.
 *   width    W in {2, 3, 4} (SSM_ERR_UNSUPPORTED otherwise)
 *   x        [batch][dim][seqlen]  in_dtype
 *   weight   [dim][width]          fp32
 *   bias     [dim] fp32, or NULL (zero)
 *   state0   [batch][dim][width-1] fp32 inputs preceding x[., ., 0], oldest
 *            first, or NULL (zeros)
 *   y        [batch][dim][seqlen]  out_dtype; must not overlap any input
 *   stateL   [batch][dim][width-1] fp32 final conv state, or NULL (not
 *            returned); may be exactly state0 (each row reads its state0
 *            before writing stateL) but must not otherwise overlap an input or y
 * Supported sizes: batch, dim, seqlen >= 1, dim <= 2^30, batch * dim * seqlen < 2^62.
 */
ssm_status_t ssm_conv1d_fwd(int batch, int dim, int seqlen, int width, ssm_dtype_t in_dtype,
                            unsigned flags, const void *x, const float *weight,
                            const float *bias, const float *state0, ssm_dtype_t out_dtype,
                            void *y, float *stateL, void *stream);

/*
 * Strided layouts for ssm_conv1d_fwd_strided: strides in ELEMENTS, time
 * contiguous.  The block's conv reads the SSM branch x, one half of the
 * input projection's [batch][2 dim][seqlen] output (glossary entry "Mamba
 * Block"), so x usually arrives as a view with rows seqlen apart and batch
 * entries 2 dim seqlen apart.
 *   x_row, y_row      distance between channel rows; >= seqlen; 0 means seqlen
 *   x_batch, y_batch  distance between batch entries; >= dim * row stride;
 *                     0 means dim * row stride
 * A stride below its minimum, a negative one, or a tensor spanning 2^56
 * elements or more is SSM_ERR_BAD_SHAPE.  Overlap is checked on each tensor's
 * address range from its first to its last element.  weight, bias and the
 * conv states stay dense.
 */
typedef struct {
    long long x_row, x_batch;
    long long y_row, y_batch;
} ssm_conv_layout_t;

/* ssm_conv1d_fwd on strided x and y: the same arguments and errors, with
 * `layout` (host pointer, read during the call only; NULL means dense). */
ssm_status_t ssm_conv1d_fwd_strided(int batch, int dim, int seqlen, int width,
                                    ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                    const float *weight, const float *bias, const float *state0,
                                    ssm_dtype_t out_dtype, void *y, float *stateL,
                                    const ssm_conv_layout_t *layout, void *stream);

/*
 * The conv on (batch, L, dim)-ordered x and y: a time step's channels
 * contiguous, time steps apart.  It is the order of the (B, L, D) tensors in
 * the reading guide's "Hardware-aware state expansion" section and the order
 * in which the input projection produces the block's x, so the conv can read
 * x as one half of a [batch][L][2 dim] projection output and feed
 * ssm_scan_fwd_bld without a transpose.
 *   x   element (b, t, d) at b * x_batch + t * x_step + d   (in_dtype)
 *   y   element (b, t, d) at b * y_batch + t * y_step + d   (out_dtype)
 *   x_step, y_step    distance between time steps; >= dim; 0 means dim
 *   x_batch, y_batch  distance between batch entries; >= seqlen * step;
 *                     0 means seqlen * step
 * Strides are in ELEMENTS of the tensor's own type.  A negative stride, one
 * below its minimum, a step stride above 2^40 or a tensor spanning 2^56
 * elements or more is SSM_ERR_BAD_SHAPE.
 */
typedef struct {
    long long x_step, x_batch;
    long long y_step, y_batch;
} ssm_conv_bld_layout_t;

/* ssm_conv1d_fwd on (batch, L, dim)-ordered x and y laid out by `layout`
 * (host pointer, read during the call only; NULL means dense): the same
 * arguments, results (bit for bit) and errors, with weight, bias and the conv
 * states dense as in ssm_conv1d_fwd ([batch][dim][width-1]); stateL may be
 * exactly state0.  Overlap is checked on address ranges from the first to
 * the last element.  Supported sizes: batch, dim, seqlen >= 1, dim <= 2^30,
 * batch * dim * seqlen < 2^62. */
ssm_status_t ssm_conv1d_fwd_bld(int batch, int dim, int seqlen, int width, ssm_dtype_t in_dtype,
                                unsigned flags, const void *x, const float *weight,
                                const float *bias, const float *state0, ssm_dtype_t out_dtype,
                                void *y, float *stateL, const ssm_conv_bld_layout_t *layout,
                                void *stream);

/*
 * One decode step: the same operation at seqlen = 1 on a persistent state.
 *   state    [batch][dim][width-1] fp32, read and overwritten in place with
 *            the window shifted by one (the new input last)
 *   x        [batch][dim] in_dtype;  weight [dim][width] fp32;  bias [dim] or NULL
 *   y        [batch][dim] out_dtype; must not overlap any input or state
 */
ssm_status_t ssm_conv1d_update(int batch, int dim, int width, ssm_dtype_t in_dtype,
                               unsigned flags, float *state, const void *x, const float *weight,
                               const float *bias, ssm_dtype_t out_dtype, void *y, void *stream);

/* ssm_conv1d_update with batch strides in ELEMENTS for x (the x half of
 * the step's [batch][2 dim] projection row, say) and y: 0 means dim, else
 * at least dim.  Errors as for ssm_conv1d_fwd_strided; the state is dense. */
ssm_status_t ssm_conv1d_update_strided(int batch, int dim, int width, ssm_dtype_t in_dtype,
                                       unsigned flags, float *state, const void *x,
                                       const float *weight, const float *bias,
                                       ssm_dtype_t out_dtype, void *y, long long x_batch,
                                       long long y_batch, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CONV_H */
