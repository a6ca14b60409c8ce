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
// (b, d)).  R = N / 4 consecutive lanes (one for N < 4) share one (b, d)
// and each owns four of its states, one 16-byte access, so every load and
// store instruction of a wave covers one contiguous kilobyte of state; the
// readout sum over n is finished across the R lanes with DPP quad permutes.
// A lane handles U (b, d) rows, U = 4 when the batch fills the GPU with one
// round of waves (else 1): the loads of all U rows are issued before the
// first row is computed, so the later rows arrive while the wave computes.
// Measured at batch 64 x dim 5120: 8.8 us per step against 10.2 us for eight
// states and one row per lane, and 9.8 us for four states and two rows;
// eight rows per lane (155 VGPRs) took 11.1 us.  The per-(b, d) scalars
// (Delta, x, z) are computed by each of the R lanes.  A, Bm and Cm come from
// cache.  The state is read with nontemporal loads and written with ordinary
// stores: with 16 layers' states rotating past the 256 MB MALL (a multi-layer
// decode) a step took 10.45 us against 11.5 us with ordinary loads, and the
// same with one state that stays in the MALL (8.9 us); nontemporal stores as
// well cost 10.6 us with the resident state, and alone 12.1 us rotating.
#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kStatesPerLane = 4;  // one 16-byte state access per row
constexpr long long kFullRoundWaves = 4096;

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

// kStream: nontemporal loads (the state, read once per token)
template <int N, bool kStream = false>
__device__ inline void load_f32(const float *p, float *v)
{
    if constexpr (N % 4 == 0) {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const f32x4 w = kStream ? __builtin_nontemporal_load(q + i) : q[i];
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

template <typename Tin, typename Tout, int N, bool kZoh, int U>
__global__ __launch_bounds__(kThreads) void state_update_kernel(UpdateParams p)
{
    constexpr int S = N < kStatesPerLane ? N : kStatesPerLane;  // states per lane
    constexpr int R = N / S;                                     // lanes per (b, d)
    constexpr int G = kThreads / R;                              // lane groups per workgroup
    // Grid: x over blocks of G * U channels, y over the batch, so the batch
    // row (and with it Bm, Cm) is uniform across the workgroup.  Row k of a
    // group is channel base + k G + group: each load instruction of the wave
    // covers contiguous rows.  Every row's loads are issued before the first
    // row is computed, so the wave's later rows arrive while it computes.
    const int b = blockIdx.y;
    const int r = threadIdx.x % R;  // which S states of the row
    const int gi = threadIdx.x / R;
    const int n0 = r * S;

    const Tin *Bp = static_cast<const Tin *>(p.Bm) + size_t(b) * size_t(p.B_b) + n0;
    const Tin *Cp = static_cast<const Tin *>(p.Cm) + size_t(b) * size_t(p.C_b) + n0;
    float bm[S], cm[S];
#pragma unroll
    for (int n = 0; n < S; ++n) {
        bm[n] = io<Tin>::load1(Bp + n);
        cm[n] = io<Tin>::load1(Cp + n);
    }

    float h[U][S], a[U][S], xv[U], dtv[U], zv[U], bias[U], skip[U];
    int dd[U];
    bool live[U];
    const bool a_vec = S % 4 == 0 && (reinterpret_cast<uintptr_t>(p.A) & 15u) == 0;
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int dk = blockIdx.x * G * U + k * G + gi;
        live[k] = dk < p.dim;
        const int d = live[k] ? dk : p.dim - 1;  // dead lanes still join the DPP sum
        dd[k] = d;
        load_f32<S, true>(p.state + (size_t(b) * p.dim + d) * N + n0, h[k]);
        const float *Ap = p.A + size_t(d) * N + n0;
        if (a_vec) {
            load_f32<S>(Ap, a[k]);
        } else {
#pragma unroll
            for (int n = 0; n < S; ++n) a[k][n] = Ap[n];
        }
        xv[k] = io<Tin>::load1(static_cast<const Tin *>(p.x) + size_t(b) * size_t(p.x_b) + d);
        dtv[k] = io<Tin>::load1(static_cast<const Tin *>(p.dt) + size_t(b) * size_t(p.dt_b) + d);
        zv[k] = p.z ? io<Tin>::load1(static_cast<const Tin *>(p.z) + size_t(b) * size_t(p.z_b) + d) : 0.0f;
        bias[k] = p.dt_bias ? p.dt_bias[d] : 0.0f;
        skip[k] = p.Dskip ? p.Dskip[d] : 0.0f;
    }

#pragma unroll
    for (int k = 0; k < U; ++k) {
        const float delta = softplus(dtv[k] + bias[k]);
        const float u = delta * xv[k];
        const float dl = delta * kLog2e;
        float acc = 0.0f;
        [[maybe_unused]] const float invd = rcp_hw(delta);
#pragma unroll
        for (int n = 0; n < S; ++n) {
            const float t = dl * a[k][n];
            const float dA = exp2_hw(t);
            float bterm = u * bm[n];
            if constexpr (kZoh) bterm *= phi_zoh(t * kLn2, dA, invd * rcp_hw(a[k][n]));
            h[k][n] = __builtin_fmaf(dA, h[k][n], bterm);
            acc = __builtin_fmaf(cm[n], h[k][n], acc);
        }
        acc = group_sum<R>(acc) + skip[k] * xv[k];
        if (p.z) acc *= silu(zv[k]);
        if (!live[k]) continue;
        float *st = p.state + (size_t(b) * p.dim + dd[k]) * N + n0;
        if constexpr (S % 4 == 0) {
#pragma unroll
            for (int i = 0; i < S / 4; ++i)
                reinterpret_cast<f32x4 *>(st)[i] =
                    f32x4{h[k][4 * i], h[k][4 * i + 1], h[k][4 * i + 2], h[k][4 * i + 3]};
        } else {
#pragma unroll
            for (int i = 0; i < S; ++i) st[i] = h[k][i];
        }
        if (r == 0) {
            const size_t yi = size_t(b) * size_t(p.y_b) + dd[k];
            if constexpr (sizeof(Tout) == 4) {
                static_cast<float *>(p.y)[yi] = acc;
            } else {
                static_cast<uint16_t *>(p.y)[yi] = uint16_t(pack_bf16x2(acc, 0.0f) & 0xffffu);
            }
        }
    }
}

template <typename Tin, typename Tout, int N, bool kZoh, int U>
hipError_t launch_rows(const UpdateArgs &a, const UpdateParams &p, hipStream_t stream)
{
    constexpr int R = N < kStatesPerLane ? 1 : N / kStatesPerLane;
    constexpr int per_block = kThreads / R * U;  // channels per workgroup
    const dim3 grid((unsigned(a.dim) + per_block - 1) / per_block, a.batch);
    if (log_enabled())
        log_line("state_update: state_update_kernel<in %s, out %s, N %d, zoh %d, rows per lane %d>, "
                 "grid (%u, %u) x %d threads", type_tag<Tin>(), type_tag<Tout>(), N, int(kZoh), U,
                 grid.x, grid.y, kThreads);
    hipLaunchKernelGGL((state_update_kernel<Tin, Tout, N, kZoh, U>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename Tin, typename Tout, int N, bool kZoh>
hipError_t launch_typed(const UpdateArgs &a, hipStream_t stream)
{
    UpdateParams p{a.batch, a.dim, a.state, a.x, a.dt, a.dt_bias, a.A,
                   a.Bm, a.Cm, a.Dskip, a.z, a.y, a.x_b, a.dt_b, a.z_b, a.y_b, a.B_b, a.C_b};
    // Four rows per lane once that still gives a full round of waves (about
    // four per SIMD of the 1024 SIMDs); smaller batches keep one row per lane
    // and with it more waves.
    constexpr int R = N < kStatesPerLane ? 1 : N / kStatesPerLane;
    const long long waves4 = (long long)a.batch * a.dim * R / (64 * 4);
    if (waves4 >= kFullRoundWaves) return launch_rows<Tin, Tout, N, kZoh, 4>(a, p, stream);
    return launch_rows<Tin, Tout, N, kZoh, 1>(a, p, stream);
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
