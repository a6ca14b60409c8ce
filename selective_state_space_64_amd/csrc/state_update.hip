// state_update.hip -- single-token decode step for gfx950.
//
// One token per sequence against a persistent fp32 state of dim x N per
// sequence, updated in place (Q&A on generation of the page "Mamba:
// Linear-Time Sequence Modeling with Selective State Spaces": a fixed-size
// state and constant work per token).  Same arithmetic as the scan at L = 1:
//     Delta = softplus(dt + dt_bias[d])
//     h[n]  = exp(Delta A[d,n]) h[n] + Delta Bm[b,n] x
//     y     = (sum_n Cm[b,n] h[n] + Dskip[d] x) * silu(z)
// (kZoh: the input term carries the exact zero-order-hold factor
// phi(Delta A) = (e^{Delta A} - 1) / (Delta A).)
//
// The step is bound by moving the state (read + write, 2 x 4N bytes per
// (b, d)).  R = N / 8 consecutive lanes share one (b, d) and each owns eight
// of its states (two 16-byte accesses in flight; four states per lane
// measured 3 % slower, sixteen 25 % slower), so a wave reads and writes
// contiguous kilobytes of state; the readout sum over n is finished across
// the R lanes with a DPP quad permute.  The per-(b, d) scalars (Delta, x, z)
// are computed by each of the R lanes.  A, Bm and Cm come from cache.
#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

constexpr int kThreads = 256;
#ifndef SSM_UPDATE_STATES
#define SSM_UPDATE_STATES 8
#endif
constexpr int kStatesPerLane = SSM_UPDATE_STATES;  // a multiple of 4 (16-byte state accesses)

struct UpdateParams {
    int batch, dim;
    float *state;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    void *y;
    // batch strides in elements of x, dt, z, y (rows of dim) and Bm, Cm (rows of N)
    long long x_b, dt_b, z_b, y_b, B_b, C_b;
};

template <int N>
__device__ inline void load_f32(const float *p, float *v)
{
    if constexpr (N % 4 == 0) {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const f32x4 w = q[i];
            v[4 * i] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = p[i];
    }
}

// Sum over groups of R consecutive lanes (R = 1, 2 or 4: within a DPP quad);
// every lane of a group gets the total.  All lanes of the wave must be active.
template <int R>
__device__ inline float group_sum(float v)
{
    if constexpr (R >= 2) {
        asm volatile("s_nop 1\n\t"
                     "v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                     : "+v"(v));
    }
    if constexpr (R >= 4) {
        asm volatile("s_nop 1\n\t"
                     "v_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                     : "+v"(v));
    }
    return v;
}

template <typename Tin, typename Tout, int N, bool kZoh>
__global__ __launch_bounds__(kThreads) void state_update_kernel(UpdateParams p)
{
    constexpr int S = N < kStatesPerLane ? N : kStatesPerLane;  // states per lane
    constexpr int R = N / S;                                     // lanes per (b, d)
    // Grid: x over channel blocks, y over the batch, so the batch row (and
    // with it Bm, Cm) is uniform across the workgroup.
    const int b = blockIdx.y;
    const int g = blockIdx.x * kThreads + threadIdx.x;
    const int r = g % R;              // which S states of the row
    const bool live = g / R < p.dim;
    const int d = live ? g / R : p.dim - 1;  // dead lanes still join the DPP sum
    const size_t idx = size_t(b) * p.dim + d;
    const int n0 = r * S;

    const Tin *Bp = static_cast<const Tin *>(p.Bm) + size_t(b) * size_t(p.B_b) + n0;
    const Tin *Cp = static_cast<const Tin *>(p.Cm) + size_t(b) * size_t(p.C_b) + n0;
    float bm[S], cm[S];
#pragma unroll
    for (int n = 0; n < S; ++n) {
        bm[n] = io<Tin>::load1(Bp + n);
        cm[n] = io<Tin>::load1(Cp + n);
    }

    float h[S], a[S];
    float *st = p.state + idx * N + n0;
    load_f32<S>(st, h);
    const float *Ap = p.A + size_t(d) * N + n0;
    if (S % 4 == 0 && (reinterpret_cast<uintptr_t>(p.A) & 15u) == 0) {
        load_f32<S>(Ap, a);
    } else {
#pragma unroll
        for (int n = 0; n < S; ++n) a[n] = Ap[n];
    }
    const float xv = io<Tin>::load1(static_cast<const Tin *>(p.x) + size_t(b) * size_t(p.x_b) + d);
    const float dtv = io<Tin>::load1(static_cast<const Tin *>(p.dt) + size_t(b) * size_t(p.dt_b) + d);
    const float bias = p.dt_bias ? p.dt_bias[d] : 0.0f;
    const float skip = p.Dskip ? p.Dskip[d] : 0.0f;

    const float delta = softplus(dtv + bias);
    const float u = delta * xv;
    const float dl = delta * kLog2e;
    float acc = 0.0f;
    [[maybe_unused]] const float invd = rcp_hw(delta);
#pragma unroll
    for (int n = 0; n < S; ++n) {
        const float t = dl * a[n];
        const float dA = exp2_hw(t);
        float bterm = u * bm[n];
        if constexpr (kZoh) bterm *= phi_zoh(t * kLn2, dA, invd * rcp_hw(a[n]));
        h[n] = __builtin_fmaf(dA, h[n], bterm);
        acc = __builtin_fmaf(cm[n], h[n], acc);
    }
    acc = group_sum<R>(acc) + skip * xv;
    if (p.z) acc *= silu(io<Tin>::load1(static_cast<const Tin *>(p.z) + size_t(b) * size_t(p.z_b) + d));
    if (!live) return;

    if constexpr (S % 4 == 0) {
#pragma unroll
        for (int i = 0; i < S / 4; ++i)
            reinterpret_cast<f32x4 *>(st)[i] = f32x4{h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i) st[i] = h[i];
    }
    if (r == 0) {
        const size_t yi = size_t(b) * size_t(p.y_b) + d;
        if constexpr (sizeof(Tout) == 4) {
            static_cast<float *>(p.y)[yi] = acc;
        } else {
            static_cast<uint16_t *>(p.y)[yi] = uint16_t(pack_bf16x2(acc, 0.0f) & 0xffffu);
        }
    }
}

template <typename Tin, typename Tout, int N, bool kZoh>
hipError_t launch_typed(const UpdateArgs &a, hipStream_t stream)
{
    UpdateParams p{a.batch, a.dim, a.state, a.x, a.dt, a.dt_bias, a.A,
                   a.Bm, a.Cm, a.Dskip, a.z, a.y, a.x_b, a.dt_b, a.z_b, a.y_b, a.B_b, a.C_b};
    constexpr int R = N < kStatesPerLane ? 1 : N / kStatesPerLane;
    dim3 grid(unsigned((size_t(a.dim) * R + kThreads - 1) / kThreads), a.batch);
    hipLaunchKernelGGL((state_update_kernel<Tin, Tout, N, kZoh>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename Tin, typename Tout, bool kZoh>
hipError_t launch_n(const UpdateArgs &a, hipStream_t stream)
{
    switch (a.dstate) {
    case 1: return launch_typed<Tin, Tout, 1, kZoh>(a, stream);
    case 2: return launch_typed<Tin, Tout, 2, kZoh>(a, stream);
    case 4: return launch_typed<Tin, Tout, 4, kZoh>(a, stream);
    case 8: return launch_typed<Tin, Tout, 8, kZoh>(a, stream);
    case 16: return launch_typed<Tin, Tout, 16, kZoh>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename Tin, typename Tout>
hipError_t launch_mode(const UpdateArgs &a, hipStream_t stream)
{
    return a.zoh ? launch_n<Tin, Tout, true>(a, stream) : launch_n<Tin, Tout, false>(a, stream);
}

}  // namespace

hipError_t launch_state_update(const UpdateArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? launch_mode<bf16_t, bf16_t>(a, stream)
                          : launch_mode<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? launch_mode<float, bf16_t>(a, stream) : launch_mode<float, float>(a, stream);
}

}  // namespace ssm
