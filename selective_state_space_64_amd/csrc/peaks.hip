// peaks.hip -- issue-rate probes for the roofline of the scan kernels.
//
// The forward scan is bound by VALU issue, and its work is a mix of plain
// fp32 ops and hardware transcendentals (v_exp_f32).  The nominal peak the
// rooflines use, 128 fp32 lanes per clock per CU, assumes packed or dual
// issue; these probes measure what the chip sustains for the instruction
// forms the kernels actually use (built, like the library, without packed
// fp32 ops):
//   kind 0  v_fma_f32: eight independent fma chains per lane
//   kind 1  v_exp_f32: eight independent exp2 chains per lane
//   kind 2  the scan's mix: per step and chain one exp2, one mul and three
//           fma (the per-element work of the recurrence: Delta*A, exp, B x,
//           state update, readout), eight chains per lane
//   kind 3  v_fma_f32 with one wave-uniform (SGPR) operand, eight chains per
//           lane: the form an operand shared by a whole wave takes
// Each lane writes one float so that nothing is optimised away.  The grid
// is sized by the caller; every access stays inside out[0 .. threads).
#include <hip/hip_runtime.h>

namespace {

constexpr int kChains = 8;
constexpr int kThreads = 256;

template <int kKind>
__global__ __launch_bounds__(kThreads) void probe_kernel(float *out, int iters, float seed,
                                                         float uniform)
{
    const int tid = blockIdx.x * kThreads + threadIdx.x;
    float a[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) a[k] = seed + 0.001f * float((threadIdx.x + k) & 15);
    // per-lane operands, so that every op reads VGPRs as in the scan kernels
    // (a literal or SGPR operand would change the instruction form)
    const float lane = 1e-9f * float(threadIdx.x & 1);
    const float m0 = 0.9999f + lane, c0 = 0.0001f + lane, m1 = -0.5f + lane, c1 = 0.25f + lane;
    const float m2 = 0.5f + lane, c2 = 0.125f + lane, m3 = 0.75f + lane, c3 = 0.0625f + lane;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) {
            if constexpr (kKind == 0) {
                a[k] = __builtin_fmaf(a[k], m0, c0);
            } else if constexpr (kKind == 1) {
                a[k] = __builtin_amdgcn_exp2f(-a[k]);  // stays in [0.5, 1]
            } else if constexpr (kKind == 3) {
                a[k] = __builtin_fmaf(a[k], uniform, c0);  // `uniform` lives in an SGPR
            } else {
                const float e = __builtin_amdgcn_exp2f(a[k] * m1);  // mul + exp
                float h = __builtin_fmaf(e, a[k], c1);              // state update
                h = __builtin_fmaf(h, m2, c2);                      // input term
                a[k] = __builtin_fmaf(h, m3, c3);                   // readout
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += a[k];
    out[tid] = s;
}

}  // namespace

extern "C" {

// Lane operations per thread of one launch of probe `kind` (0..3) with
// `iters` iterations: instructions of the measured form, per lane.
long long ssm_peaks_ops_per_thread(int kind, int iters)
{
    const long long per = kind == 2 ? 5 : 1;  // kind 2: exp, mul, 3 fma per chain step
    return per * kChains * (long long)iters;
}

// Launch probe `kind` on `stream` with `blocks` workgroups of 256 threads;
// `out` must hold blocks * 256 floats.  Returns 0, or -1 for an unknown kind
// or a non-positive size, or the HIP error code of the launch.
int ssm_peaks_launch(int kind, int blocks, int iters, float *out, void *stream)
{
    if (blocks < 1 || iters < 1 || !out) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
    case 0: hipLaunchKernelGGL(probe_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, out, iters, 0.5f, 0.9999f); break;
    case 1: hipLaunchKernelGGL(probe_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, out, iters, 0.5f, 0.9999f); break;
    case 2: hipLaunchKernelGGL(probe_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, out, iters, 0.5f, 0.9999f); break;
    case 3: hipLaunchKernelGGL(probe_kernel<3>, dim3(blocks), dim3(kThreads), 0, s, out, iters, 0.5f, 0.9999f); break;
    default: return -1;
    }
    return int(hipGetLastError());
}

}  // extern "C"
