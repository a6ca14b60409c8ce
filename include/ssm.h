/*
 * ssm.h -- C ABI of the MI355X (gfx950) selective state-space (S6) library.
 *
 * Two operations, both from the page "Mamba: Linear-Time Sequence Modeling
 * with Selective State Spaces" (reading guide to arXiv 2312.00752):
 *
 *   ssm_scan_fwd      the fused selective scan over a whole sequence
 *                     (ssm_scan_fwd_strided: the same on strided views).
 *                     "Method": A-bar = exp(Delta A) by zero-order hold; the
 *                     recurrence h_t = A-bar_t h_{t-1} + B-bar_t x_t; the
 *                     readout y_t = C_t h_t taken after the step-t update.
 *                     "The selection mechanism (S6)": Delta_t, B_t, C_t
 *                     depend on the token; Delta_t = softplus(dt + dt_bias).
 *                     "Hardware-aware state expansion": the expanded
 *                     (batch, L, dim, N) state is never written to memory;
 *                     only the contracted output and the final state are.
 *                     B-bar follows the simplified form dB = Delta * B of the
 *                     dynamic-parameterization section of the page
 *                     "Mamba选择性状态空间机制：效率提升10倍的核心突破", or,
 *                     with SSM_FLAG_ZOH_B, the exact zero-order-hold form.
 *                     Output: y = (C . h + Dskip * x) * silu(z), silu(z) =
 *                     z * sigmoid(z); a NULL z means no gate.
 *
 *   ssm_state_update  one decode step: the same arithmetic at L = 1 on a
 *                     fixed dim x N state per sequence, updated in place
 *                     (Q&A on generation: constant work per token, no KV cache).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     densely packed (last index fastest), except where a layout argument
 *     gives strides.  The library allocates nothing,
 *     keeps no state between calls, and is reentrant.
 *   - Layouts: x, dt, z, y      [batch][dim][seqlen]
 *              Bm, Cm           [batch][dstate][seqlen]
 *              A                [dim][dstate]          (fp32, real, diagonal)
 *              Dskip, dt_bias   [dim]                  (fp32)
 *              h0, hL, state    [batch][dim][dstate]   (fp32)
 *     For ssm_state_update the seqlen index is dropped: x, dt, z, y are
 *     [batch][dim] and Bm, Cm are [batch][dstate].
 *   - in_dtype is the storage type of x, dt, z, Bm, Cm; arithmetic is fp32.
 *   - Every pointer must be aligned to its element size (2 bytes for bf16,
 *     4 for fp32); the decode `state` must be 16-byte aligned.  The kernels
 *     use 16-byte vector accesses wherever the addresses allow it.
 *   - Argument errors are found before anything is launched: the call then
 *     returns the status and writes nothing.  A failed launch returns
 *     SSM_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation of `stream`.
 *   - Calls are asynchronous: they return once the work is enqueued on
 *     `stream` (a hipStream_t; NULL is the default stream).
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 1

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL_ARG = 1,    /* a required pointer is NULL                         */
    SSM_ERR_BAD_SHAPE = 2,   /* a size < 1 or beyond the supported range (below)    */
    SSM_ERR_BAD_DTYPE = 3,   /* in_dtype or out_dtype is not a value of ssm_dtype_t */
    SSM_ERR_MISALIGNED = 4,  /* a pointer below its element alignment (state: 16 B) */
    SSM_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap    */
    SSM_ERR_UNSUPPORTED = 6, /* dstate not in {1,2,4,8,16}, or an unknown flag bit   */
    SSM_ERR_WORKSPACE = 7,   /* workspace smaller than ssm_scan_fwd_workspace_bytes */
    SSM_ERR_HIP = 8          /* the HIP runtime rejected the launch                */
} ssm_status_t;

/* flags bit 0: use the exact zero-order-hold B-bar of the "Method" section,
 * B-bar = (Delta A)^-1 (exp(Delta A) - 1) Delta B, instead of Delta B. */
#define SSM_FLAG_ZOH_B 0x1u

/* flags bit 1 (ssm_scan_fwd, with either form of B-bar, and ssm_scan_bwd):
 * checkpoints for the backward pass.  The backward recomputes the scan's
 * states from the state entering every 64-step chunk ("Hardware-aware state
 * expansion": states are recomputed, not stored).  With this bit,
 * ssm_scan_fwd writes those checkpoints into `workspace`, which must then be
 * at least ssm_scan_bwd_workspace_bytes(...) bytes (see ssm_bwd.h), and
 * ssm_scan_bwd given the same workspace reads them instead of running its own
 * recomputation pass.  The forward's other outputs are unchanged bit for bit.
 * Any other flag bit is SSM_ERR_UNSUPPORTED. */
#define SSM_FLAG_CHECKPOINTS 0x2u

/* SSM_ABI_VERSION of the loaded library. */
int ssm_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *ssm_status_string(ssm_status_t status);

/* Device workspace ssm_scan_fwd needs for these sizes, in bytes (0: none;
 * the workspace argument may then be NULL).  It is non-zero when the
 * sequence is split into segments scanned in parallel, which the library
 * does when batch x ceil(dim / 16) is small (under 256) and seqlen long
 * (segments of at least 1024 steps, a multiple of 256).  The recurrence is
 * affine in the state,
 * so each segment but the last first runs from a zero state (h0 for the
 * first) to get its end state and Delta sum; the main pass then enters
 * segment s with the earlier segments composed,
 *     h <- exp(A sum_s Delta) h + (end state of s),
 * the composition of the scan's associative operator over whole segments
 * (the "Parallel Associative Scan" glossary entry of the reading-guide page).
 * The workspace holds, per segment and (batch, channel), dstate + 1 floats.
 * A function of the sizes only; invalid sizes give 0. */
size_t ssm_scan_fwd_workspace_bytes(int batch, int dim, int seqlen, int dstate);

/*
 * Selective scan over the whole sequence.
 *   x        [batch][dim][seqlen]   in_dtype  input
 *   dt       [batch][dim][seqlen]   in_dtype  raw step, before bias and softplus
 *   dt_bias  [dim]     fp32, or NULL (zero): Delta = softplus(dt + dt_bias)
 *   A        [dim][dstate]          fp32      diagonal state matrix per channel
 *   Bm, Cm   [batch][dstate][seqlen] in_dtype input and output matrices,
 *                                              shared by all channels
 *   Dskip    [dim]     fp32, or NULL (zero)   skip weight
 *   z        [batch][dim][seqlen]   in_dtype, or NULL (no gate)
 *   h0       [batch][dim][dstate]   fp32, or NULL (zero initial state)
 *   y        [batch][dim][seqlen]   out_dtype output; must not overlap any input
 *   hL       [batch][dim][dstate]   fp32 final state, or NULL (not returned);
 *            may be exactly h0 (each channel reads its h0 before writing hL)
 *            but must not otherwise overlap an input or y
 *   workspace, workspace_bytes: device scratch of at least
 *            ssm_scan_fwd_workspace_bytes(...) bytes (NULL allowed when 0),
 *            4-byte aligned, overlapping no input or output; its contents
 *            are scratch before and after the call;
 *            with SSM_FLAG_CHECKPOINTS, the backward pass's workspace (at
 *            least ssm_scan_bwd_workspace_bytes(...) bytes), which receives
 *            the checkpoints and must not overlap any input or output
 * Supported sizes: batch <= 65535, dim <= 2^30, seqlen <= 2^28 - 4096,
 * dstate in {1, 2, 4, 8, 16}.
 */
ssm_status_t ssm_scan_fwd(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype,
                          unsigned flags, const void *x, const void *dt, const float *dt_bias,
                          const float *A, const void *Bm, const void *Cm, const float *Dskip,
                          const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                          float *hL, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Strided layouts for ssm_scan_fwd_strided.  The Mamba block (glossary entry
 * "Mamba Block" of the same reading-guide page) feeds the scan from one input
 * projection that yields both the SSM branch x and the gate z, so the two
 * usually arrive as halves of one [batch][2 dim][seqlen] buffer; Bm and Cm
 * likewise as parts of one projection.  These strides let such views be
 * passed without a copy.  All strides are in ELEMENTS of the tensor's own
 * type; time is always the contiguous index (stride 1).
 *   seq_row        distance between consecutive channels (rows) of x, dt, z
 *                  and y, shared by the four; >= seqlen; 0 means seqlen
 *   seq_batch[4]   distance between batch entries of x, dt, z, y (in that
 *                  order); each >= dim * seq_row; 0 means dim * seq_row
 *   bc_row         distance between consecutive states of Bm and Cm; >= seqlen;
 *                  0 means seqlen
 *   bc_batch[2]    distance between batch entries of Bm, Cm; each >=
 *                  dstate * bc_row; 0 means dstate * bc_row
 * Strides of 0 everywhere (or a NULL layout) give the dense layout of
 * ssm_scan_fwd.  Each row start is aligned like any other element; the
 * kernels still use 16-byte vector accesses when the strides keep rows on
 * 16-byte boundaries.  A negative stride, one below its minimum, seq_row or
 * bc_row above 2^28 - 4096, or a tensor spanning 2^56 elements or more is
 * SSM_ERR_BAD_SHAPE.
 */
typedef struct {
    long long seq_row;
    long long seq_batch[4];
    long long bc_row;
    long long bc_batch[2];
} ssm_scan_layout_t;

/*
 * ssm_scan_fwd on strided inputs and output: the same arguments, flags and
 * errors, with `layout` (host pointer, read during the call only; NULL means
 * dense) giving the strides of x, dt, z, y, Bm and Cm.  A, Dskip, dt_bias, h0,
 * hL and the checkpoints stay dense.  Overlap is checked on address ranges: y
 * and hL must not overlap the range from the first to the last element of any
 * input (as laid out by the strides), so y may not be interleaved with an
 * input even where no element coincides.
 */
ssm_status_t ssm_scan_fwd_strided(int batch, int dim, int seqlen, int dstate,
                                  ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                                  float *hL, void *workspace, size_t workspace_bytes,
                                  const ssm_scan_layout_t *layout, void *stream);

/*
 * ssm_scan_fwd_strided without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call itself allocates nothing either.
 * Where ssm_scan_fwd_workspace_bytes(...) is non-zero (a sequence split), the
 * split's planes go to a scratch array inside the library: one copy per GPU,
 * 17 825 792 bytes (16384 x 16 x 17 floats), held from the library's first
 * use on that GPU until the process ends.  Every split shape fits in it (the
 * split makes segments x batch x dim at most 16384 x 16); a shape that did
 * not would be SSM_ERR_WORKSPACE.  All calls on one GPU share that GPU's array:
 * calls that overlap in time on the same GPU (on other streams or from other
 * threads) race on it and must be serialised by the caller.  Nothing in it
 * needs clearing between calls.  `stream` must belong to the current device.
 * Arguments, layout, results and errors are those of ssm_scan_fwd_strided,
 * except that SSM_FLAG_CHECKPOINTS (which needs the backward pass's
 * workspace) is SSM_ERR_UNSUPPORTED.  The device address of the array is
 * looked up on the first call on each device; a failure there is SSM_ERR_HIP.
 * Results equal those of ssm_scan_fwd_strided bit for bit (same kernels).
 */
ssm_status_t ssm_scan_fwd_noalloc(int batch, int dim, int seqlen, int dstate,
                                  ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                                  float *hL, const ssm_scan_layout_t *layout, void *stream);

/*
 * The selective scan on tensors in (batch, L, dim) order: a time step's
 * channels contiguous, time steps apart.  It is the order of the (B, L, D)
 * output in the reading guide's "Hardware-aware state expansion" section and
 * the order in which a model's input projection produces x and z, so those
 * can be passed without a transpose (x and z as the two halves of one
 * [batch][L][2 dim] projection output).
 *   x, dt, z, y  element (b, t, d) at b * *_batch + t * *_step + d
 *   Bm, Cm       element (b, t, n) at b * *_batch + t * *_step + n
 *   A, Dskip, dt_bias, h0, hL as in ssm_scan_fwd (dense).
 * Strides are in ELEMENTS of the tensor's own type; the channel (state)
 * index is always contiguous.
 *   x_step .. y_step   distance between time steps of x, dt, z, y; >= dim;
 *                      0 means dim
 *   x_batch .. y_batch distance between batch entries; >= seqlen * step;
 *                      0 means seqlen * step
 *   B_step, C_step     distance between time steps of Bm, Cm; >= dstate;
 *                      0 means dstate
 *   B_batch, C_batch   >= seqlen * step; 0 means seqlen * step
 * A NULL layout means all zero (dense (batch, L, dim) and (batch, L, dstate)).
 * A negative stride, one below its minimum, a step stride above 2^40 or a
 * tensor spanning 2^56 elements or more is SSM_ERR_BAD_SHAPE.
 */
typedef struct {
    long long x_step, dt_step, z_step, y_step;
    long long x_batch, dt_batch, z_batch, y_batch;
    long long B_step, C_step, B_batch, C_batch;
} ssm_bld_layout_t;

/* Device workspace ssm_scan_fwd_bld needs, in bytes (never 0 for valid
 * sizes; 0 for sizes it refuses).  The kernels run channels along the lanes
 * of a wave and cut the sequence into pieces walked by separate waves, so
 * that enough waves run at once; the workspace holds, per piece and
 * (batch, channel), the piece's map h -> exp(A sum Delta) h + e (dstate + 1
 * floats), then the state entering it, composed in order with the scan's
 * associative operator (the "Parallel Associative Scan" glossary entry). */
size_t ssm_scan_fwd_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate);

/*
 * ssm_scan_fwd on (batch, L, dim)-ordered tensors, laid out by `layout`
 * (host pointer, read during the call only).  Same arguments, results (up to
 * the association order of the fp32 sums) and errors as ssm_scan_fwd, with:
 *   workspace, workspace_bytes: at least ssm_scan_fwd_bld_workspace_bytes(...)
 *            bytes, 4-byte aligned, overlapping no input or output (required)
 *   flags:   SSM_FLAG_ZOH_B only (SSM_FLAG_CHECKPOINTS, whose checkpoints
 *            feed the [batch][dim][L] backward pass, is SSM_ERR_UNSUPPORTED)
 * Overlap is checked on address ranges from the first to the last element.
 * Supported sizes: as ssm_scan_fwd.
 */
ssm_status_t ssm_scan_fwd_bld(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype,
                              unsigned flags, const void *x, const void *dt, const float *dt_bias,
                              const float *A, const void *Bm, const void *Cm, const float *Dskip,
                              const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                              float *hL, void *workspace, size_t workspace_bytes,
                              const ssm_bld_layout_t *layout, void *stream);

/*
 * One decode step (seqlen = 1) on a persistent state.
 *   state    [batch][dim][dstate]   fp32, read and overwritten in place
 *   x, dt    [batch][dim]           in_dtype
 *   dt_bias  [dim] fp32 or NULL;  A [dim][dstate] fp32
 *   Bm, Cm   [batch][dstate]        in_dtype
 *   Dskip    [dim] fp32 or NULL;  z [batch][dim] in_dtype or NULL
 *   y        [batch][dim]           out_dtype; must not overlap any input or state
 * Supported sizes: batch <= 65535, dim <= 2^30, dstate in {1, 2, 4, 8, 16}.
 */
ssm_status_t ssm_state_update(int batch, int dim, int dstate, ssm_dtype_t in_dtype,
                              unsigned flags, float *state, const void *x, const void *dt,
                              const float *dt_bias, const float *A, const void *Bm,
                              const void *Cm, const float *Dskip, const void *z,
                              ssm_dtype_t out_dtype, void *y, void *stream);

/*
 * Per-token inputs of the decode step usually arrive as slices of the
 * step's projection outputs: x and z as the halves of one [batch][2 dim]
 * row (glossary entry "Mamba Block"), Bm and Cm as parts of one
 * [batch][dt_rank + 2 dstate] row.  Batch strides in ELEMENTS (0 means
 * dense: dim for x, dt, z, y; dstate for Bm, Cm); each at least that dense
 * value.  A negative stride, one below its minimum, or a tensor spanning 2^56
 * elements or more is SSM_ERR_BAD_SHAPE; overlap is checked on address
 * ranges from first to last element.
 */
typedef struct {
    long long x_batch, dt_batch, z_batch, y_batch;
    long long B_batch, C_batch;
} ssm_update_layout_t;

/* ssm_state_update on batch-strided inputs and output: the same arguments
 * and errors, with `layout` (host pointer, read during the call only; NULL
 * means dense).  The state stays dense. */
ssm_status_t ssm_state_update_strided(int batch, int dim, int dstate, ssm_dtype_t in_dtype,
                                      unsigned flags, float *state, const void *x,
                                      const void *dt, const float *dt_bias, const float *A,
                                      const void *Bm, const void *Cm, const float *Dskip,
                                      const void *z, ssm_dtype_t out_dtype, void *y,
                                      const ssm_update_layout_t *layout, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
