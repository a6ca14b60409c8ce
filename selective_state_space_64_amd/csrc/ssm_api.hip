// ssm_api.hip -- the C ABI declared in include/ssm.h: argument validation
// and dispatch to the gfx950 kernels.  Every argument error is detected here,
// before anything is enqueued, so a failing call has no side effects.
#include "ssm.h"
#include "ssm_bwd.h"
#include "ssm_conv.h"

#include <stdint.h>
#include <string.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "ssm_launch.hpp"

namespace {

// True when p is not a multiple of `align` bytes (NULL is never misaligned).
bool misaligned(const void *p, uintptr_t align)
{
    return p && (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0;
}

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void *p, size_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}

bool overlaps(const void *p, size_t pb, const void *q, size_t qb)
{
    if (!p || !q || pb == 0 || qb == 0) return false;
    const Span a = span(p, pb), b = span(q, qb);
    return a.lo < b.hi && b.lo < a.hi;
}

// The value of an enum argument as the int a C caller passed: its bits are
// read without loading the argument as the enum type, so a value outside the
// enumeration (an error the validation reports) is not undefined behaviour.
template <typename E>
int enum_bits(const E &e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v = 0;
    memcpy(&v, &e, sizeof v);
    return v;
}

bool valid_dtype(int t) { return t == SSM_F32 || t == SSM_BF16; }
size_t dsize(int t) { return t == SSM_BF16 ? 2 : 4; }
bool valid_dstate(int n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

// Product of positive ints as size_t, or 0 on overflow past 2^62.
size_t mul3(long long a, long long b, long long c)
{
    const unsigned __int128 r = (unsigned __int128)a * (unsigned __int128)b * (unsigned __int128)c;
    if (r > ((unsigned __int128)1 << 62)) return 0;
    return size_t(r);
}

// Row stride of strided [batch][rows][seqlen] tensors: 0 means seqlen;
// false when below seqlen or beyond the kernels' 32-bit in-wave offsets.
bool row_stride(long long given, int seqlen, long long &rs)
{
    rs = given ? given : seqlen;
    return rs >= seqlen && rs <= ssm::kMaxSeqlen;
}

// Batch stride (0 means rows * rs) and span in elements, from the first to
// one past the last element, of a [batch][rows][seqlen] tensor whose rows
// are rs apart; false when the stride is negative or below rows * rs, or the
// span reaches 2^56 elements.
bool batch_span(long long given, int batch, int rows, long long rs, int seqlen, long long &sb,
                size_t &sp)
{
    sb = given ? given : rows * rs;
    if (sb < rows * rs) return false;
    const __int128 n = (__int128)(batch - 1) * sb + (__int128)(rows - 1) * rs + seqlen;
    if (n >= ((__int128)1 << 56)) return false;
    sp = size_t(n);
    return true;
}

// Device scratch of ssm_scan_fwd_noalloc: a file-scope array, one copy per
// GPU (held from the library's first use on that GPU until the process
// ends).  It holds the sequence split's planes, at most kScratchBytes: the
// split gives at most kSplitTargetWgs / (batch * ceil(dim / 16)) segments, so
// segments x batch x dim <= kSplitTargetWgs * 16, times (dstate + 1) <= 17
// floats (17 825 792 bytes for 16384 workgroups).  In host code
// the array's name is only a stand-in for the symbol; its device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// ever handed to a kernel.  Every call on a GPU shares that GPU's copy, so
// calls that overlap in time on one GPU (other streams, other threads) race
// on it.  Nothing in it needs clearing between calls: the aggregate pass
// writes every plane the main pass reads.
constexpr size_t kScratchBytes = size_t(ssm::kSplitTargetWgs) * 16 * 17 * sizeof(float);
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
hipError_t scratch_address(float **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float *>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

// Step and batch strides (0 = dense) and the span in elements of a
// (batch, seqlen, rowlen) tensor whose row index is contiguous: false when a
// stride is negative or below its minimum, or the span reaches 2^56.
bool bld_span(long long given_step, long long given_batch, int batch, int seqlen, int rowlen,
              long long &st, long long &sb, size_t &sp)
{
    st = given_step ? given_step : rowlen;
    if (st < rowlen || st > (1ll << 40)) return false;
    const __int128 min_b = (__int128)seqlen * st;
    sb = given_batch ? given_batch : (long long)min_b;
    if ((__int128)sb < min_b) return false;
    const __int128 n = (__int128)(batch - 1) * sb + (__int128)(seqlen - 1) * st + rowlen;
    if (n >= ((__int128)1 << 56)) return false;
    sp = size_t(n);
    return true;
}

// ssm_scan_fwd_strided, and with noalloc set ssm_scan_fwd_noalloc: the
// split's planes then go to the library's own scratch array instead of the
// caller's workspace (which must be NULL), and checkpoints are refused.
ssm_status_t scan_fwd_impl(int batch, int dim, int seqlen, int dstate, int in_dtype,
                           unsigned flags, const void *x, const void *dt, const float *dt_bias,
                           const float *A, const void *Bm, const void *Cm, const float *Dskip,
                           const void *z, const float *h0, int out_dtype, void *y,
                           float *hL, void *workspace, size_t workspace_bytes,
                           const ssm_scan_layout_t *layout, void *stream, bool noalloc)
{
    if (!x || !dt || !A || !Bm || !Cm || !y) return SSM_ERR_NULL_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen)
        return SSM_ERR_BAD_SHAPE;
    if (!valid_dstate(dstate) || (flags & ~(SSM_FLAG_ZOH_B | SSM_FLAG_CHECKPOINTS)) != 0)
        return SSM_ERR_UNSUPPORTED;
    if (noalloc && (flags & SSM_FLAG_CHECKPOINTS)) return SSM_ERR_UNSUPPORTED;

    const size_t st_elems = mul3(batch, dim, dstate);
    if (!mul3(batch, dim, seqlen) || !mul3(batch, dstate, seqlen) || !st_elems)
        return SSM_ERR_BAD_SHAPE;
    const ssm_scan_layout_t dense{};
    const ssm_scan_layout_t &lay = layout ? *layout : dense;
    // Strides with defaults filled in, and each tensor's span in elements.
    long long row, bc_row, seq_b[4], bc_b[2];
    size_t seq_span[4], bc_span[2];
    if (!row_stride(lay.seq_row, seqlen, row) || !row_stride(lay.bc_row, seqlen, bc_row))
        return SSM_ERR_BAD_SHAPE;
    for (int i = 0; i < 4; ++i)
        if (!batch_span(lay.seq_batch[i], batch, dim, row, seqlen, seq_b[i], seq_span[i]))
            return SSM_ERR_BAD_SHAPE;
    for (int i = 0; i < 2; ++i)
        if (!batch_span(lay.bc_batch[i], batch, dstate, bc_row, seqlen, bc_b[i], bc_span[i]))
            return SSM_ERR_BAD_SHAPE;
    const bool ckpt = (flags & SSM_FLAG_CHECKPOINTS) != 0;
    const size_t split_bytes = ssm::scan_fwd_split_bytes(batch, dim, seqlen, dstate);
    // Bytes of the workspace this call uses: the backward pass's workspace
    // with checkpoints (the split's planes then follow the checkpoints),
    // otherwise the split's planes, if any.
    const size_t ws_bytes = noalloc ? 0
                            : ckpt  ? ssm::scan_bwd_workspace_bytes(batch, dim, seqlen, dstate)
                                    : split_bytes;
    if (ckpt && !workspace) return SSM_ERR_NULL_ARG;
    if (noalloc && split_bytes > kScratchBytes) return SSM_ERR_WORKSPACE;

    const size_t in = dsize(in_dtype);
    for (const void *p : {x, dt, Bm, Cm, z})
        if (misaligned(p, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)dt_bias, (const void *)A, (const void *)Dskip,
                          (const void *)h0, (const void *)hL})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (misaligned(y, dsize(out_dtype))) return SSM_ERR_MISALIGNED;
    if (ws_bytes && misaligned(workspace, 4)) return SSM_ERR_MISALIGNED;

    const size_t ybytes = seq_span[3] * dsize(out_dtype);
    const size_t hbytes = st_elems * sizeof(float);
    if (workspace_bytes < ws_bytes || (ws_bytes && !workspace)) return SSM_ERR_WORKSPACE;
    struct In {
        const void *p;
        size_t bytes;
    } inputs[] = {{x, seq_span[0] * in}, {dt, seq_span[1] * in},    {dt_bias, dim * sizeof(float)},
                  {A, size_t(dim) * dstate * sizeof(float)},
                  {Bm, bc_span[0] * in}, {Cm, bc_span[1] * in},     {Dskip, dim * sizeof(float)},
                  {z, seq_span[2] * in}, {h0, hbytes}};
    for (const In &i : inputs) {
        if (overlaps(y, ybytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        // hL may be exactly h0 (read before written per channel), nothing else
        if (hL && !(i.p == h0 && hL == h0) && overlaps(hL, hbytes, i.p, i.bytes))
            return SSM_ERR_ALIAS;
        if (overlaps(workspace, ws_bytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
    }
    if (overlaps(y, ybytes, hL, hbytes)) return SSM_ERR_ALIAS;
    if (overlaps(workspace, ws_bytes, y, ybytes) || overlaps(workspace, ws_bytes, hL, hbytes))
        return SSM_ERR_ALIAS;

    float *ws = static_cast<float *>(workspace);
    const size_t ck_floats = ssm::scan_checkpoint_floats(batch, dim, seqlen, dstate);
    float *agg = split_bytes ? (ckpt ? ws + ck_floats : ws) : nullptr;
    if (noalloc) {
        float *own = nullptr;
        if (scratch_address(&own) != hipSuccess) return SSM_ERR_HIP;
        agg = split_bytes ? own : nullptr;
    }
    ssm::ScanArgs a{batch, dim, seqlen, dstate, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                    (flags & SSM_FLAG_ZOH_B) != 0, x, dt, dt_bias, A, Bm, Cm, Dskip, z, h0, y, hL,
                    ckpt ? ws : nullptr,
                    row, seq_b[0], seq_b[1], seq_b[2], seq_b[3], bc_row, bc_b[0], bc_b[1], agg, 0};
    const hipError_t e = ssm::launch_scan_fwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

namespace ssm {

bool log_enabled()
{
    static const bool on = [] {
        const char *v = getenv("SSM_LOG");
        return v && *v && !(v[0] == '0' && v[1] == 0);
    }();
    return on;
}

void log_line(const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    fprintf(stderr, "[ssm] %s\n", buf);
}

}  // namespace ssm

extern "C" {

// Implementations behind the entry points, dtype arguments as int.
static ssm_status_t ssm_state_update_strided_impl(int batch, int dim, int dstate, int in_dtype,
                                      unsigned flags, float *state, const void *x,
                                      const void *dt, const float *dt_bias, const float *A,
                                      const void *Bm, const void *Cm, const float *Dskip,
                                      const void *z, int out_dtype, void *y,
                                      const ssm_update_layout_t *layout, void *stream);
static ssm_status_t ssm_conv1d_fwd_strided_impl(int batch, int dim, int seqlen, int width,
                                    int in_dtype, unsigned flags, const void *x,
                                    const float *weight, const float *bias, const float *state0,
                                    int out_dtype, void *y, float *stateL,
                                    const ssm_conv_layout_t *layout, void *stream);
static ssm_status_t ssm_conv1d_update_strided_impl(int batch, int dim, int width, int in_dtype,
                                       unsigned flags, float *state, const void *x,
                                       const float *weight, const float *bias,
                                       int out_dtype, void *y, long long x_batch,
                                       long long y_batch, void *stream);
static ssm_status_t ssm_scan_bwd_strided_impl(int batch, int dim, int seqlen, int dstate,
                                  int in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, int grad_dtype,
                                  const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                                  float *dBm, float *dCm, float *dA, float *dDskip,
                                  float *ddt_bias, float *dh0, void *workspace,
                                  size_t workspace_bytes, const ssm_scan_bwd_layout_t *layout,
                                  void *stream);


int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char *ssm_status_string(ssm_status_t status)
{
    // C callers may pass any int; reading the argument's bits as an int keeps
    // a value outside the enumeration defined behaviour here
    int s = 0;
    memcpy(&s, &status, sizeof s);
    switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case SSM_ERR_BAD_SHAPE: return "batch, dim and seqlen must be >= 1 and within the supported range";
    case SSM_ERR_BAD_DTYPE: return "in_dtype/out_dtype must be SSM_F32 or SSM_BF16";
    case SSM_ERR_MISALIGNED: return "a pointer is not aligned to its element size (state: 16 bytes)";
    case SSM_ERR_ALIAS: return "an output buffer overlaps an input it must not overlap";
    case SSM_ERR_UNSUPPORTED:
        return "unsupported dstate (1, 2, 4, 8 or 16) or conv width (2, 3 or 4), or an unknown flag bit";
    case SSM_ERR_WORKSPACE: return "workspace smaller than the documented size for this call";
    case SSM_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    }
    return "unknown status";
}

size_t ssm_scan_fwd_workspace_bytes(int batch, int dim, int seqlen, int dstate)
{
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen || !valid_dstate(dstate))
        return 0;
    return ssm::scan_fwd_split_bytes(batch, dim, seqlen, dstate);
}

ssm_status_t ssm_scan_fwd(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype,
                          unsigned flags, const void *x, const void *dt, const float *dt_bias,
                          const float *A, const void *Bm, const void *Cm, const float *Dskip,
                          const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                          float *hL, void *workspace, size_t workspace_bytes, void *stream)
{
    return scan_fwd_impl(batch, dim, seqlen, dstate, enum_bits(in_dtype), flags, x, dt, dt_bias, A,
                         Bm, Cm, Dskip, z, h0, enum_bits(out_dtype), y, hL, workspace,
                         workspace_bytes, nullptr, stream, false);
}

ssm_status_t ssm_scan_fwd_strided(int batch, int dim, int seqlen, int dstate,
                                  ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                                  float *hL, void *workspace, size_t workspace_bytes,
                                  const ssm_scan_layout_t *layout, void *stream)
{
    return scan_fwd_impl(batch, dim, seqlen, dstate, enum_bits(in_dtype), flags, x, dt, dt_bias, A,
                         Bm, Cm, Dskip, z, h0, enum_bits(out_dtype), y, hL, workspace,
                         workspace_bytes, layout, stream, false);
}

ssm_status_t ssm_scan_fwd_noalloc(int batch, int dim, int seqlen, int dstate,
                                  ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, ssm_dtype_t out_dtype, void *y,
                                  float *hL, const ssm_scan_layout_t *layout, void *stream)
{
    return scan_fwd_impl(batch, dim, seqlen, dstate, enum_bits(in_dtype), flags, x, dt, dt_bias, A,
                         Bm, Cm, Dskip, z, h0, enum_bits(out_dtype), y, hL, nullptr, 0, layout,
                         stream, true);
}

size_t ssm_scan_fwd_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate)
{
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen || !valid_dstate(dstate))
        return 0;
    return ssm::scan_bld_workspace_bytes(batch, dim, seqlen, dstate);
}

ssm_status_t ssm_scan_fwd_bld(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype_e,
                              unsigned flags, const void *x, const void *dt, const float *dt_bias,
                              const float *A, const void *Bm, const void *Cm, const float *Dskip,
                              const void *z, const float *h0, ssm_dtype_t out_dtype_e, void *y,
                              float *hL, void *workspace, size_t workspace_bytes,
                              const ssm_bld_layout_t *layout, void *stream)
{
    const int in_dtype = enum_bits(in_dtype_e), out_dtype = enum_bits(out_dtype_e);
    if (!x || !dt || !A || !Bm || !Cm || !y || !workspace) return SSM_ERR_NULL_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen)
        return SSM_ERR_BAD_SHAPE;
    if (!valid_dstate(dstate) || (flags & ~SSM_FLAG_ZOH_B) != 0) return SSM_ERR_UNSUPPORTED;
    const size_t st_elems = mul3(batch, dim, dstate);
    if (!mul3(batch, dim, seqlen) || !mul3(batch, dstate, seqlen) || !st_elems)
        return SSM_ERR_BAD_SHAPE;
    const ssm_bld_layout_t dense{};
    const ssm_bld_layout_t &lay = layout ? *layout : dense;
    // x, dt, z, y, then Bm, Cm: strides with defaults filled in, spans
    const long long gs[6] = {lay.x_step, lay.dt_step, lay.z_step, lay.y_step, lay.B_step,
                             lay.C_step};
    const long long gb[6] = {lay.x_batch, lay.dt_batch, lay.z_batch, lay.y_batch, lay.B_batch,
                             lay.C_batch};
    long long st[6], sb[6];
    size_t sp[6];
    for (int i = 0; i < 6; ++i)
        if (!bld_span(gs[i], gb[i], batch, seqlen, i < 4 ? dim : dstate, st[i], sb[i], sp[i]))
            return SSM_ERR_BAD_SHAPE;
    const size_t ws_bytes = ssm::scan_bld_workspace_bytes(batch, dim, seqlen, dstate);

    const size_t in = dsize(in_dtype);
    for (const void *p : {x, dt, Bm, Cm, z})
        if (misaligned(p, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)dt_bias, (const void *)A, (const void *)Dskip,
                          (const void *)h0, (const void *)hL, (const void *)workspace})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (misaligned(y, dsize(out_dtype))) return SSM_ERR_MISALIGNED;
    if (workspace_bytes < ws_bytes) return SSM_ERR_WORKSPACE;

    const size_t ybytes = sp[3] * dsize(out_dtype);
    const size_t hbytes = st_elems * sizeof(float);
    struct In {
        const void *p;
        size_t bytes;
    } inputs[] = {{x, sp[0] * in},     {dt, sp[1] * in},     {dt_bias, dim * sizeof(float)},
                  {A, size_t(dim) * dstate * sizeof(float)},
                  {Bm, sp[4] * in},    {Cm, sp[5] * in},     {Dskip, dim * sizeof(float)},
                  {z, sp[2] * in},     {h0, hbytes}};
    for (const In &i : inputs) {
        if (overlaps(y, ybytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        if (hL && !(i.p == h0 && hL == h0) && overlaps(hL, hbytes, i.p, i.bytes))
            return SSM_ERR_ALIAS;
        if (overlaps(workspace, ws_bytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
    }
    if (overlaps(y, ybytes, hL, hbytes)) return SSM_ERR_ALIAS;
    if (overlaps(workspace, ws_bytes, y, ybytes) || overlaps(workspace, ws_bytes, hL, hbytes))
        return SSM_ERR_ALIAS;

    ssm::BldArgs a{batch, dim, seqlen, dstate, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                   (flags & SSM_FLAG_ZOH_B) != 0, x, dt, dt_bias, A, Bm, Cm, Dskip, z, h0, y, hL,
                   st[0], sb[0], st[1], sb[1], st[2], sb[2], st[3], sb[3], st[4], sb[4], st[5],
                   sb[5], static_cast<float *>(workspace)};
    const hipError_t e = ssm::launch_scan_bld(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_state_update(int batch, int dim, int dstate, ssm_dtype_t in_dtype,
                              unsigned flags, float *state, const void *x, const void *dt,
                              const float *dt_bias, const float *A, const void *Bm,
                              const void *Cm, const float *Dskip, const void *z,
                              ssm_dtype_t out_dtype, void *y, void *stream)
{
    return ssm_state_update_strided_impl(batch, dim, dstate, enum_bits(in_dtype), flags, state, x,
                                         dt, dt_bias, A, Bm, Cm, Dskip, z, enum_bits(out_dtype), y,
                                         nullptr, stream);
}

static ssm_status_t ssm_state_update_strided_impl(int batch, int dim, int dstate, int in_dtype,
                                      unsigned flags, float *state, const void *x,
                                      const void *dt, const float *dt_bias, const float *A,
                                      const void *Bm, const void *Cm, const float *Dskip,
                                      const void *z, int out_dtype, void *y,
                                      const ssm_update_layout_t *layout, void *stream)
{
    if (!state || !x || !dt || !A || !Bm || !Cm || !y) return SSM_ERR_NULL_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || dim > ssm::kMaxDim) return SSM_ERR_BAD_SHAPE;
    if (!valid_dstate(dstate) || (flags & ~SSM_FLAG_ZOH_B) != 0) return SSM_ERR_UNSUPPORTED;

    const size_t rows = mul3(batch, dim, 1);
    if (batch > ssm::kMaxBatch || dim > ssm::kMaxDim) return SSM_ERR_BAD_SHAPE;
    const size_t st_elems = mul3(batch, dim, dstate);
    if (!rows || !st_elems) return SSM_ERR_BAD_SHAPE;
    const ssm_update_layout_t dense{};
    const ssm_update_layout_t &lay = layout ? *layout : dense;
    // batch strides and spans: x, dt, z, y (rows of dim), Bm, Cm (rows of dstate)
    long long sb[6];
    size_t sp[6];
    const long long given[6] = {lay.x_batch, lay.dt_batch, lay.z_batch, lay.y_batch, lay.B_batch,
                                lay.C_batch};
    for (int i = 0; i < 6; ++i) {
        const int n = i < 4 ? dim : dstate;
        if (!batch_span(given[i], batch, 1, n, n, sb[i], sp[i])) return SSM_ERR_BAD_SHAPE;
    }

    const size_t in = dsize(in_dtype);
    if (misaligned(state, 16)) return SSM_ERR_MISALIGNED;
    for (const void *p : {x, dt, Bm, Cm, z})
        if (misaligned(p, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)dt_bias, (const void *)A, (const void *)Dskip})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (misaligned(y, dsize(out_dtype))) return SSM_ERR_MISALIGNED;

    const size_t ybytes = sp[3] * dsize(out_dtype);
    const size_t sbytes = st_elems * sizeof(float);
    struct In {
        const void *p;
        size_t bytes;
    } inputs[] = {{x, sp[0] * in},
                  {dt, sp[1] * in},
                  {dt_bias, dim * sizeof(float)},
                  {A, size_t(dim) * dstate * sizeof(float)},
                  {Bm, sp[4] * in},
                  {Cm, sp[5] * in},
                  {Dskip, dim * sizeof(float)},
                  {z, sp[2] * in}};
    for (const In &i : inputs) {
        if (overlaps(y, ybytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        if (overlaps(state, sbytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
    }
    if (overlaps(y, ybytes, state, sbytes)) return SSM_ERR_ALIAS;

    ssm::UpdateArgs a{batch, dim, dstate, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                      (flags & SSM_FLAG_ZOH_B) != 0, state, x, dt, dt_bias, A, Bm, Cm, Dskip, z, y,
                      sb[0], sb[1], sb[2], sb[3], sb[4], sb[5]};
    const hipError_t e = ssm::launch_state_update(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_state_update_strided(int batch, int dim, int dstate, ssm_dtype_t in_dtype,
                                      unsigned flags, float *state, const void *x,
                                      const void *dt, const float *dt_bias, const float *A,
                                      const void *Bm, const void *Cm, const float *Dskip,
                                      const void *z, ssm_dtype_t out_dtype, void *y,
                                      const ssm_update_layout_t *layout, void *stream)
{
    return ssm_state_update_strided_impl(batch, dim, dstate, enum_bits(in_dtype), flags, state, x,
                                         dt, dt_bias, A, Bm, Cm, Dskip, z, enum_bits(out_dtype), y,
                                         layout, stream);
}

ssm_status_t ssm_conv1d_fwd(int batch, int dim, int seqlen, int width, ssm_dtype_t in_dtype,
                            unsigned flags, const void *x, const float *weight,
                            const float *bias, const float *state0, ssm_dtype_t out_dtype,
                            void *y, float *stateL, void *stream)
{
    return ssm_conv1d_fwd_strided_impl(batch, dim, seqlen, width, enum_bits(in_dtype), flags, x,
                                       weight, bias, state0, enum_bits(out_dtype), y, stateL,
                                       nullptr, stream);
}

static ssm_status_t ssm_conv1d_fwd_strided_impl(int batch, int dim, int seqlen, int width,
                                    int in_dtype, unsigned flags, const void *x,
                                    const float *weight, const float *bias, const float *state0,
                                    int out_dtype, void *y, float *stateL,
                                    const ssm_conv_layout_t *layout, void *stream)
{
    if (!x || !weight || !y) return SSM_ERR_NULL_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || seqlen < 1 || dim > ssm::kMaxDim) return SSM_ERR_BAD_SHAPE;
    if (width < 2 || width > 4 || (flags & ~SSM_CONV_SILU) != 0) return SSM_ERR_UNSUPPORTED;
    const size_t st_elems = mul3(batch, dim, width - 1);
    if (!mul3(batch, dim, seqlen) || !st_elems) return SSM_ERR_BAD_SHAPE;
    const ssm_conv_layout_t dense{};
    const ssm_conv_layout_t &lay = layout ? *layout : dense;
    long long x_row = lay.x_row ? lay.x_row : seqlen, y_row = lay.y_row ? lay.y_row : seqlen;
    long long x_b, y_b;
    size_t x_span, y_span;
    if (x_row < seqlen || y_row < seqlen ||
        !batch_span(lay.x_batch, batch, dim, x_row, seqlen, x_b, x_span) ||
        !batch_span(lay.y_batch, batch, dim, y_row, seqlen, y_b, y_span))
        return SSM_ERR_BAD_SHAPE;

    const size_t in = dsize(in_dtype);
    if (misaligned(x, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)weight, (const void *)bias, (const void *)state0,
                          (const void *)stateL})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (misaligned(y, dsize(out_dtype))) return SSM_ERR_MISALIGNED;

    const size_t ybytes = y_span * dsize(out_dtype);
    const size_t sbytes = st_elems * sizeof(float);
    struct In {
        const void *p;
        size_t bytes;
    } inputs[] = {{x, x_span * in},
                  {weight, size_t(dim) * width * sizeof(float)},
                  {bias, dim * sizeof(float)},
                  {state0, sbytes}};
    for (const In &i : inputs) {
        if (overlaps(y, ybytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        // stateL may be exactly state0 (read before written per row), nothing else
        if (stateL && !(i.p == state0 && stateL == state0) && overlaps(stateL, sbytes, i.p, i.bytes))
            return SSM_ERR_ALIAS;
    }
    if (overlaps(y, ybytes, stateL, sbytes)) return SSM_ERR_ALIAS;

    ssm::ConvArgs a{batch, dim, seqlen, width, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                    (flags & SSM_CONV_SILU) != 0, x, weight, bias, state0, y, stateL,
                    x_row, x_b, y_row, y_b};
    const hipError_t e = ssm::launch_conv1d_fwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_conv1d_fwd_strided(int batch, int dim, int seqlen, int width,
                                    ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                    const float *weight, const float *bias, const float *state0,
                                    ssm_dtype_t out_dtype, void *y, float *stateL,
                                    const ssm_conv_layout_t *layout, void *stream)
{
    return ssm_conv1d_fwd_strided_impl(batch, dim, seqlen, width, enum_bits(in_dtype), flags, x,
                                       weight, bias, state0, enum_bits(out_dtype), y, stateL,
                                       layout, stream);
}

ssm_status_t ssm_conv1d_fwd_bld(int batch, int dim, int seqlen, int width, ssm_dtype_t in_dtype_e,
                                unsigned flags, const void *x, const float *weight,
                                const float *bias, const float *state0, ssm_dtype_t out_dtype_e,
                                void *y, float *stateL, const ssm_conv_bld_layout_t *layout,
                                void *stream)
{
    const int in_dtype = enum_bits(in_dtype_e), out_dtype = enum_bits(out_dtype_e);
    if (!x || !weight || !y) return SSM_ERR_NULL_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || seqlen < 1 || dim > ssm::kMaxDim) return SSM_ERR_BAD_SHAPE;
    if (width < 2 || width > 4 || (flags & ~SSM_CONV_SILU) != 0) return SSM_ERR_UNSUPPORTED;
    const size_t st_elems = mul3(batch, dim, width - 1);
    if (!mul3(batch, dim, seqlen) || !st_elems) return SSM_ERR_BAD_SHAPE;
    const ssm_conv_bld_layout_t dense{};
    const ssm_conv_bld_layout_t &lay = layout ? *layout : dense;
    long long x_t, x_b, y_t, y_b;
    size_t x_span, y_span;
    if (!bld_span(lay.x_step, lay.x_batch, batch, seqlen, dim, x_t, x_b, x_span) ||
        !bld_span(lay.y_step, lay.y_batch, batch, seqlen, dim, y_t, y_b, y_span))
        return SSM_ERR_BAD_SHAPE;

    const size_t in = dsize(in_dtype);
    if (misaligned(x, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)weight, (const void *)bias, (const void *)state0,
                          (const void *)stateL})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (misaligned(y, dsize(out_dtype))) return SSM_ERR_MISALIGNED;

    const size_t ybytes = y_span * dsize(out_dtype);
    const size_t sbytes = st_elems * sizeof(float);
    struct In {
        const void *p;
        size_t bytes;
    } inputs[] = {{x, x_span * in},
                  {weight, size_t(dim) * width * sizeof(float)},
                  {bias, dim * sizeof(float)},
                  {state0, sbytes}};
    for (const In &i : inputs) {
        if (overlaps(y, ybytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        // stateL may be exactly state0 (read before written per row), nothing else
        if (stateL && !(i.p == state0 && stateL == state0) && overlaps(stateL, sbytes, i.p, i.bytes))
            return SSM_ERR_ALIAS;
    }
    if (overlaps(y, ybytes, stateL, sbytes)) return SSM_ERR_ALIAS;

    ssm::ConvBldArgs a{batch, dim, seqlen, width, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                       (flags & SSM_CONV_SILU) != 0, x, weight, bias, state0, y, stateL,
                       x_t, x_b, y_t, y_b};
    const hipError_t e = ssm::launch_conv1d_bld(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_conv1d_update(int batch, int dim, int width, ssm_dtype_t in_dtype,
                               unsigned flags, float *state, const void *x, const float *weight,
                               const float *bias, ssm_dtype_t out_dtype, void *y, void *stream)
{
    return ssm_conv1d_update_strided_impl(batch, dim, width, enum_bits(in_dtype), flags, state, x,
                                          weight, bias, enum_bits(out_dtype), y, 0, 0, stream);
}

static ssm_status_t ssm_conv1d_update_strided_impl(int batch, int dim, int width, int in_dtype,
                                       unsigned flags, float *state, const void *x,
                                       const float *weight, const float *bias,
                                       int out_dtype, void *y, long long x_batch,
                                       long long y_batch, void *stream)
{
    if (!state || !x || !weight || !y) return SSM_ERR_NULL_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || dim > ssm::kMaxDim) return SSM_ERR_BAD_SHAPE;
    if (width < 2 || width > 4 || (flags & ~SSM_CONV_SILU) != 0) return SSM_ERR_UNSUPPORTED;
    const size_t rows = mul3(batch, dim, 1);
    const size_t st_elems = mul3(batch, dim, width - 1);
    if (!rows || !st_elems) return SSM_ERR_BAD_SHAPE;
    long long x_b, y_b;
    size_t x_span, y_span;
    if (!batch_span(x_batch, batch, 1, dim, dim, x_b, x_span) ||
        !batch_span(y_batch, batch, 1, dim, dim, y_b, y_span))
        return SSM_ERR_BAD_SHAPE;

    const size_t in = dsize(in_dtype);
    if (misaligned(x, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)state, (const void *)weight, (const void *)bias})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (misaligned(y, dsize(out_dtype))) return SSM_ERR_MISALIGNED;

    const size_t ybytes = y_span * dsize(out_dtype);
    const size_t sbytes = st_elems * sizeof(float);
    struct In {
        const void *p;
        size_t bytes;
    } inputs[] = {{x, x_span * in},
                  {weight, size_t(dim) * width * sizeof(float)},
                  {bias, dim * sizeof(float)}};
    for (const In &i : inputs) {
        if (overlaps(y, ybytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        if (overlaps(state, sbytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
    }
    if (overlaps(y, ybytes, state, sbytes)) return SSM_ERR_ALIAS;

    ssm::ConvUpdateArgs a{batch, dim, width, in_dtype == SSM_BF16, out_dtype == SSM_BF16,
                          (flags & SSM_CONV_SILU) != 0, state, x, weight, bias, y, x_b, y_b};
    const hipError_t e = ssm::launch_conv1d_update(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_conv1d_update_strided(int batch, int dim, int width, ssm_dtype_t in_dtype,
                                       unsigned flags, float *state, const void *x,
                                       const float *weight, const float *bias,
                                       ssm_dtype_t out_dtype, void *y, long long x_batch,
                                       long long y_batch, void *stream)
{
    return ssm_conv1d_update_strided_impl(batch, dim, width, enum_bits(in_dtype), flags, state, x,
                                          weight, bias, enum_bits(out_dtype), y, x_batch, y_batch,
                                          stream);
}

size_t ssm_scan_bwd_workspace_bytes(int batch, int dim, int seqlen, int dstate)
{
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen || !valid_dstate(dstate))
        return 0;
    return ssm::scan_bwd_workspace_bytes(batch, dim, seqlen, dstate);
}

ssm_status_t ssm_scan_bwd(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype,
                          unsigned flags, const void *x, const void *dt, const float *dt_bias,
                          const float *A, const void *Bm, const void *Cm, const float *Dskip,
                          const void *z, const float *h0, ssm_dtype_t grad_dtype,
                          const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                          float *dBm, float *dCm, float *dA, float *dDskip, float *ddt_bias,
                          float *dh0, void *workspace, size_t workspace_bytes, void *stream)
{
    return ssm_scan_bwd_strided_impl(batch, dim, seqlen, dstate, enum_bits(in_dtype), flags, x, dt,
                                     dt_bias, A, Bm, Cm, Dskip, z, h0, enum_bits(grad_dtype), dy,
                                     dhL, dx, ddt, dz, dBm, dCm, dA, dDskip, ddt_bias, dh0,
                                     workspace, workspace_bytes, nullptr, stream);
}

static ssm_status_t ssm_scan_bwd_strided_impl(int batch, int dim, int seqlen, int dstate,
                                  int in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, int grad_dtype,
                                  const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                                  float *dBm, float *dCm, float *dA, float *dDskip,
                                  float *ddt_bias, float *dh0, void *workspace,
                                  size_t workspace_bytes, const ssm_scan_bwd_layout_t *layout,
                                  void *stream)
{
    if (!x || !dt || !A || !Bm || !Cm || !dy || !dx || !ddt || !dBm || !dCm || !dA)
        return SSM_ERR_NULL_ARG;
    if (z && !dz) return SSM_ERR_NULL_ARG;
    if (!z) dz = nullptr;
    if (!valid_dtype(in_dtype) || !valid_dtype(grad_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen)
        return SSM_ERR_BAD_SHAPE;
    if (!valid_dstate(dstate) || (flags & ~(SSM_FLAG_CHECKPOINTS | SSM_FLAG_ZOH_B)) != 0)
        return SSM_ERR_UNSUPPORTED;

    const size_t bc_elems = mul3(batch, dstate, seqlen);
    const size_t st_elems = mul3(batch, dim, dstate);
    if (!mul3(batch, dim, seqlen) || !bc_elems || !st_elems) return SSM_ERR_BAD_SHAPE;
    const ssm_scan_bwd_layout_t dense{};
    const ssm_scan_bwd_layout_t &lay = layout ? *layout : dense;
    // x, dt, z, dy, dx, ddt, dz: strides and spans in elements; Bm, Cm likewise
    long long row, bc_row, seq_b[7], bc_b[2];
    size_t sp[7], bc_span[2];
    if (!row_stride(lay.seq_row, seqlen, row) || !row_stride(lay.bc_row, seqlen, bc_row))
        return SSM_ERR_BAD_SHAPE;
    for (int i = 0; i < 7; ++i)
        if (!batch_span(lay.seq_batch[i], batch, dim, row, seqlen, seq_b[i], sp[i]))
            return SSM_ERR_BAD_SHAPE;
    for (int i = 0; i < 2; ++i)
        if (!batch_span(lay.bc_batch[i], batch, dstate, bc_row, seqlen, bc_b[i], bc_span[i]))
            return SSM_ERR_BAD_SHAPE;
    const size_t ws_need = ssm_scan_bwd_workspace_bytes(batch, dim, seqlen, dstate);
    if (!workspace && ws_need) return SSM_ERR_NULL_ARG;

    const size_t in = dsize(in_dtype), gs = dsize(grad_dtype);
    for (const void *p : {x, dt, Bm, Cm, z})
        if (misaligned(p, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {dy, (const void *)dx, (const void *)ddt, (const void *)dz})
        if (misaligned(p, gs)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)dt_bias, (const void *)A, (const void *)Dskip,
                          (const void *)h0, (const void *)dhL, (const void *)dBm, (const void *)dCm,
                          (const void *)dA, (const void *)dDskip, (const void *)ddt_bias,
                          (const void *)dh0, (const void *)workspace})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;

    if (workspace_bytes < ws_need) return SSM_ERR_WORKSPACE;

    struct Buf {
        const void *p;
        size_t bytes;
    };
    const size_t fb = sizeof(float);
    const Buf inputs[] = {{x, sp[0] * in},  {dt, sp[1] * in},  {dt_bias, dim * fb},
                          {A, size_t(dim) * dstate * fb},
                          {Bm, bc_span[0] * in},  {Cm, bc_span[1] * in},  {Dskip, dim * fb},
                          {z, sp[2] * in},  {h0, st_elems * fb},  {dy, sp[3] * gs},
                          {dhL, st_elems * fb}};
    const Buf outputs[] = {{dx, sp[4] * gs},         {ddt, sp[5] * gs},       {dz, sp[6] * gs},
                           {dBm, bc_elems * fb},     {dCm, bc_elems * fb},
                           {dA, size_t(dim) * dstate * fb},
                           {dDskip, dim * fb},       {ddt_bias, dim * fb},    {dh0, st_elems * fb},
                           {workspace, ws_need}};
    const int nout = int(sizeof(outputs) / sizeof(outputs[0]));
    for (int o = 0; o < nout; ++o) {
        for (const Buf &i : inputs)
            if (overlaps(outputs[o].p, outputs[o].bytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        for (int o2 = o + 1; o2 < nout; ++o2)
            if (overlaps(outputs[o].p, outputs[o].bytes, outputs[o2].p, outputs[o2].bytes))
                return SSM_ERR_ALIAS;
    }
    ssm::BwdArgs a{batch, dim, seqlen, dstate, in_dtype == SSM_BF16, grad_dtype == SSM_BF16,
                   x, dt, dt_bias, A, Bm, Cm, Dskip, z, h0, dy, dhL, dx, ddt, dz, dBm, dCm, dA,
                   dDskip, ddt_bias, dh0, workspace, (flags & SSM_FLAG_CHECKPOINTS) != 0,
                   row, seq_b[0], seq_b[1], seq_b[2], seq_b[3], seq_b[4], seq_b[5], seq_b[6],
                   bc_row, bc_b[0], bc_b[1], (flags & SSM_FLAG_ZOH_B) != 0};
    const hipError_t e = ssm::launch_scan_bwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_scan_bwd_strided(int batch, int dim, int seqlen, int dstate,
                                  ssm_dtype_t in_dtype, unsigned flags, const void *x,
                                  const void *dt, const float *dt_bias, const float *A,
                                  const void *Bm, const void *Cm, const float *Dskip,
                                  const void *z, const float *h0, ssm_dtype_t grad_dtype,
                                  const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                                  float *dBm, float *dCm, float *dA, float *dDskip,
                                  float *ddt_bias, float *dh0, void *workspace,
                                  size_t workspace_bytes, const ssm_scan_bwd_layout_t *layout,
                                  void *stream)
{
    return ssm_scan_bwd_strided_impl(batch, dim, seqlen, dstate, enum_bits(in_dtype), flags, x, dt,
                                     dt_bias, A, Bm, Cm, Dskip, z, h0, enum_bits(grad_dtype), dy,
                                     dhL, dx, ddt, dz, dBm, dCm, dA, dDskip, ddt_bias, dh0,
                                     workspace, workspace_bytes, layout, stream);
}

size_t ssm_scan_bwd_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate)
{
    if (!ssm_scan_bwd_workspace_bytes(batch, dim, seqlen, dstate)) return 0;
    return ssm::scan_bwd_bld_workspace_bytes(batch, dim, seqlen, dstate);
}

ssm_status_t ssm_scan_bwd_bld(int batch, int dim, int seqlen, int dstate, ssm_dtype_t in_dtype_e,
                              unsigned flags, const void *x, const void *dt, const float *dt_bias,
                              const float *A, const void *Bm, const void *Cm, const float *Dskip,
                              const void *z, const float *h0, ssm_dtype_t grad_dtype_e,
                              const void *dy, const float *dhL, void *dx, void *ddt, void *dz,
                              float *dBm, float *dCm, float *dA, float *dDskip, float *ddt_bias,
                              float *dh0, void *workspace, size_t workspace_bytes,
                              const ssm_scan_bwd_bld_layout_t *layout, void *stream)
{
    const int in_dtype = enum_bits(in_dtype_e), grad_dtype = enum_bits(grad_dtype_e);
    if (!x || !dt || !A || !Bm || !Cm || !dy || !dx || !ddt || !dBm || !dCm || !dA || !workspace)
        return SSM_ERR_NULL_ARG;
    if (z && !dz) return SSM_ERR_NULL_ARG;
    if (!z) dz = nullptr;
    if (!valid_dtype(in_dtype) || !valid_dtype(grad_dtype)) return SSM_ERR_BAD_DTYPE;
    if (batch < 1 || dim < 1 || seqlen < 1 || batch > ssm::kMaxBatch || dim > ssm::kMaxDim ||
        seqlen > ssm::kMaxSeqlen)
        return SSM_ERR_BAD_SHAPE;
    if (!valid_dstate(dstate) || (flags & ~SSM_FLAG_ZOH_B) != 0) return SSM_ERR_UNSUPPORTED;
    const size_t bc_elems = mul3(batch, dstate, seqlen);
    const size_t st_elems = mul3(batch, dim, dstate);
    if (!mul3(batch, dim, seqlen) || !bc_elems || !st_elems) return SSM_ERR_BAD_SHAPE;
    const ssm_scan_bwd_bld_layout_t dense{};
    const ssm_scan_bwd_bld_layout_t &lay = layout ? *layout : dense;
    // x, dt, z, dy, dx, ddt, dz, then Bm, Cm: strides with defaults filled in, spans
    long long st[9], sb[9];
    size_t sp[9];
    for (int i = 0; i < 7; ++i)
        if (!bld_span(lay.step[i], lay.batch_stride[i], batch, seqlen, dim, st[i], sb[i], sp[i]))
            return SSM_ERR_BAD_SHAPE;
    if (!bld_span(lay.B_step, lay.B_batch, batch, seqlen, dstate, st[7], sb[7], sp[7]) ||
        !bld_span(lay.C_step, lay.C_batch, batch, seqlen, dstate, st[8], sb[8], sp[8]))
        return SSM_ERR_BAD_SHAPE;
    const size_t ws_need = ssm::scan_bwd_bld_workspace_bytes(batch, dim, seqlen, dstate);
    if (!ws_need) return SSM_ERR_BAD_SHAPE;  // a workspace of 2^62 bytes or more

    const size_t in = dsize(in_dtype), gs = dsize(grad_dtype);
    for (const void *p : {x, dt, Bm, Cm, z})
        if (misaligned(p, in)) return SSM_ERR_MISALIGNED;
    for (const void *p : {dy, (const void *)dx, (const void *)ddt, (const void *)dz})
        if (misaligned(p, gs)) return SSM_ERR_MISALIGNED;
    for (const void *p : {(const void *)dt_bias, (const void *)A, (const void *)Dskip,
                          (const void *)h0, (const void *)dhL, (const void *)dBm, (const void *)dCm,
                          (const void *)dA, (const void *)dDskip, (const void *)ddt_bias,
                          (const void *)dh0, (const void *)workspace})
        if (misaligned(p, 4)) return SSM_ERR_MISALIGNED;
    if (workspace_bytes < ws_need) return SSM_ERR_WORKSPACE;

    struct Buf {
        const void *p;
        size_t bytes;
    };
    const size_t fb = sizeof(float);
    const Buf inputs[] = {{x, sp[0] * in},  {dt, sp[1] * in},  {dt_bias, dim * fb},
                          {A, size_t(dim) * dstate * fb},
                          {Bm, sp[7] * in},  {Cm, sp[8] * in},  {Dskip, dim * fb},
                          {z, sp[2] * in},  {h0, st_elems * fb},  {dy, sp[3] * gs},
                          {dhL, st_elems * fb}};
    const Buf outputs[] = {{dx, sp[4] * gs},         {ddt, sp[5] * gs},       {dz, sp[6] * gs},
                           {dBm, bc_elems * fb},     {dCm, bc_elems * fb},
                           {dA, size_t(dim) * dstate * fb},
                           {dDskip, dim * fb},       {ddt_bias, dim * fb},    {dh0, st_elems * fb},
                           {workspace, ws_need}};
    const int nout = int(sizeof(outputs) / sizeof(outputs[0]));
    for (int o = 0; o < nout; ++o) {
        for (const Buf &i : inputs)
            if (overlaps(outputs[o].p, outputs[o].bytes, i.p, i.bytes)) return SSM_ERR_ALIAS;
        for (int o2 = o + 1; o2 < nout; ++o2)
            if (overlaps(outputs[o].p, outputs[o].bytes, outputs[o2].p, outputs[o2].bytes))
                return SSM_ERR_ALIAS;
    }
    ssm::BwdBldArgs a{batch, dim, seqlen, dstate, in_dtype == SSM_BF16, grad_dtype == SSM_BF16,
                      (flags & SSM_FLAG_ZOH_B) != 0, x, dt, dt_bias, A, Bm, Cm, Dskip, z, h0, dy,
                      dhL, dx, ddt, dz, dBm, dCm, dA, dDskip, ddt_bias, dh0, workspace,
                      {st[0], st[1], st[2], st[3], st[4], st[5], st[6]},
                      {sb[0], sb[1], sb[2], sb[3], sb[4], sb[5], sb[6]},
                      st[7], sb[7], st[8], sb[8]};
    const hipError_t e = ssm::launch_scan_bwd_bld(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
