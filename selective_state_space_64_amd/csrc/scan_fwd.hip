// scan_fwd.hip -- fused selective-scan forward pass for gfx950.
//
// Computes, per (batch b, channel d), over t = 0..L-1
// ("Method" and "The selection mechanism (S6)" sections of the page
// "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"):
//     Delta_t = softplus(dt_t + dt_bias[d])
//     h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t Bm[b,n,t] x_t
//     y_t     = (sum_n Cm[b,n,t] h_t[n] + Dskip[d] x_t) * silu(z_t)
// with the state expansion kept on chip ("Hardware-aware state expansion"):
// only y and the final state are written to HBM.
//
// Work split.  A workgroup of 4 waves owns one batch row and 16 channels.
// Each 16-lane DPP row of a wave owns one channel; lane j of the row owns the
// K consecutive timesteps [l0 + jK, l0 + jK + K) of a chunk of 16K timesteps.
// The workgroup walks the sequence chunk by chunk.  For each state n:
//   1. each lane folds its K steps into one affine map h -> a h + b
//      (a = exp2(A' sum Delta), b by a K-step fma chain),
//   2. a 4-level DPP row scan composes the 16 maps (the associative scan of
//      "Hardware-aware state expansion"; the chunking follows the soft186.com
//      page's chunked-computation section),
//   3. each lane applies its prefix to the carry entering the chunk and
//      replays its K steps, accumulating C_t h_t into y_t,
//   4. the row's last lane publishes the carry for the next chunk in LDS.
// Bm and Cm chunks (shared by every channel of the batch row) are staged once
// per workgroup into LDS as fp32, double-buffered, one barrier per chunk.
// No MFMA: the recurrence is not a dense contraction.
#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

constexpr int kRow = 16;                    // lanes per channel (one DPP row)
constexpr int kWaves = 4;                   // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kChannels = kThreads / kRow;  // channels per workgroup

struct ScanParams {
    int dim, seqlen;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    void *y;
    float *hL;
};

__device__ inline bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Inclusive scan of affine maps h -> a h + b over the 16 lanes of each DPP
// row, then the state at the end (hend) and at the start (hin) of every
// lane's block given the state `carry` entering the chunk.  Level s combines
// lane j with lane j - s, whose map covers earlier steps and is applied
// first: (a, b) <- (a_{j-s} a, b_{j-s} a + b).  Lanes with no partner inside
// the row are left unwritten (bound_ctrl off), i.e. combined with the
// identity map.  Lane 0 of each row keeps hin = carry.
// Each v_*_dpp reads its DPP source at least two wait states after that
// register was last written (the GFX9 VALU-write -> DPP-read hazard), hence
// the s_nop padding.  All 64 lanes must be active.
__device__ inline void row_scan(float &a, float &b, float carry, float &hend, float &hin)
{
    hin = carry;
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 0\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 0\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 0\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fma_f32 %2, %0, %4, %1\n\t"
        "s_nop 1\n\t"
        "v_mov_b32_dpp %3, %2 row_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(a), "+v"(b), "=&v"(hend), "+v"(hin)
        : "v"(carry));
}

template <typename Tout, int K>
__device__ inline void store_y(Tout *dst, bool vec, int count, const float *v)
{
    if constexpr (sizeof(Tout) == 4) {
        if (vec) {
            f32x4 *q = reinterpret_cast<f32x4 *>(dst);
#pragma unroll
            for (int i = 0; i < K / 4; ++i) {
                f32x4 w = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
                __builtin_nontemporal_store(w, q + i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < K; ++i)
                if (i < count) reinterpret_cast<float *>(dst)[i] = v[i];
        }
    } else {
        if (vec) {
            u32x4 *q = reinterpret_cast<u32x4 *>(dst);
#pragma unroll
            for (int i = 0; i < K / 8; ++i) {
                u32x4 w;
                w.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
                w.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
                w.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
                w.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
                __builtin_nontemporal_store(w, q + i);
            }
        } else {
            uint16_t *s = reinterpret_cast<uint16_t *>(dst);
#pragma unroll
            for (int i = 0; i < K; ++i)
                if (i < count) s[i] = uint16_t(pack_bf16x2(v[i], 0.0f) & 0xffffu);
        }
    }
}

template <typename Tin, typename Tout, int N, int K>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(ScanParams p)
{
    static_assert(K % 8 == 0, "K must be a multiple of 8");
    static_assert(N * kRow <= kThreads, "one staging slot per thread");
    constexpr int T = kRow * K;  // timesteps per chunk
    constexpr int Q = K / 4;     // float4 per lane per state

    // Bm/Cm chunk in LDS, fp32, layout [n][q][lane j] of float4 so that the
    // 16 lanes of a row read 256 contiguous bytes per ds_read_b128.
    __shared__ float4 sB[2][N * Q * kRow];
    __shared__ float4 sC[2][N * Q * kRow];
    __shared__ float sA[kChannels * N];      // A * log2(e)
    __shared__ float sCarry[kChannels * N];  // state entering the current chunk

    const int tid = threadIdx.x;
    const int j = tid & (kRow - 1);
    const int c = tid / kRow;
    const int b = blockIdx.y;
    const int dim = p.dim;
    const int L = p.seqlen;
    const int d = blockIdx.x * kChannels + c;
    const bool live = d < dim;
    const int dc = live ? d : dim - 1;

    const size_t row = (size_t(b) * dim + dc) * size_t(L);
    const Tin *xr = static_cast<const Tin *>(p.x) + row;
    const Tin *dtr = static_cast<const Tin *>(p.dt) + row;
    const Tin *zr = p.z ? static_cast<const Tin *>(p.z) + row : nullptr;
    const Tin *Bb = static_cast<const Tin *>(p.Bm) + size_t(b) * N * L;
    const Tin *Cb = static_cast<const Tin *>(p.Cm) + size_t(b) * N * L;

    for (int s = tid; s < kChannels * N; s += kThreads) {
        const int cc = s / N, n = s % N;
        const int dd = min(int(blockIdx.x) * kChannels + cc, dim - 1);
        sA[s] = p.A[size_t(dd) * N + n] * kLog2e;
    }
    if (j == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            sCarry[c * N + n] = p.h0 ? p.h0[(size_t(b) * dim + dc) * N + n] : 0.0f;
    }
    const float bias = p.dt_bias ? p.dt_bias[dc] : 0.0f;
    const float skip = p.Dskip ? p.Dskip[dc] : 0.0f;

    // staging slot of this thread: state sn, lane block sj
    const bool stager = tid < N * kRow;
    const int sn = tid / kRow, sj = tid % kRow;
    raw_run<Tin, K> stB, stC;
    auto stage_load = [&](int chunk) {
        const int l = chunk * T + sj * K;
        const int cnt = max(0, min(K, L - l));
        const Tin *pb = Bb + size_t(sn) * L + l;
        const Tin *pc = Cb + size_t(sn) * L + l;
        load_raw<Tin, K>(pb, cnt == K && aligned16(pb), cnt, stB);
        load_raw<Tin, K>(pc, cnt == K && aligned16(pc), cnt, stC);
    };
    auto stage_store = [&](int buf) {
        float vb[K], vc[K];
        decode_raw<Tin, K>(stB, vb);
        decode_raw<Tin, K>(stC, vc);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            sB[buf][(sn * Q + q) * kRow + sj] =
                make_float4(vb[4 * q], vb[4 * q + 1], vb[4 * q + 2], vb[4 * q + 3]);
            sC[buf][(sn * Q + q) * kRow + sj] =
                make_float4(vc[4 * q], vc[4 * q + 1], vc[4 * q + 2], vc[4 * q + 3]);
        }
    };

    raw_run<Tin, K> rx, rdt, rz;
    auto xdz_load = [&](int chunk) {
        const int l = chunk * T + j * K;
        const int cnt = max(0, min(K, L - l));
        const bool vec = cnt == K && aligned16(xr + l) && aligned16(dtr + l);
        load_raw<Tin, K>(xr + l, vec, cnt, rx);
        load_raw<Tin, K>(dtr + l, vec, cnt, rdt);
        if (zr) load_raw<Tin, K>(zr + l, cnt == K && aligned16(zr + l), cnt, rz);
    };

    const int nchunks = (L + T - 1) / T;
    if (stager) {
        stage_load(0);
        stage_store(0);
    }
    xdz_load(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        const int l0 = ch * T + j * K;
        const int cnt = max(0, min(K, L - l0));

        // Delta, Delta*x and the skip term for this lane's K steps; steps past
        // the end of the sequence get Delta = 0 (identity map: a = 1, b = 0).
        float delta[K], u[K], yv[K];
        float sumd = 0.0f;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const float xv = decode_raw_at<Tin, K>(rx, i);
            const float dv = softplus(decode_raw_at<Tin, K>(rdt, i) + bias);
            const bool in = i < cnt;
            delta[i] = in ? dv : 0.0f;
            u[i] = in ? dv * xv : 0.0f;
            yv[i] = skip * xv;
            sumd += delta[i];
        }
        raw_run<Tin, K> zc;
        if (zr) zc = rz;
        if (ch + 1 < nchunks) {
            xdz_load(ch + 1);
            if (stager) stage_load(ch + 1);
        }

        // LDS operands of state n are loaded one iteration ahead.
        auto load_state = [&](int n, float *v, const float4 *src) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float4 w = src[(n * Q + q) * kRow + j];
                v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
            }
        };
        float bv[K];
        load_state(0, bv, sB[buf]);
        float ap = sA[c * N];
        float carry = sCarry[c * N];
#pragma unroll 1
        for (int n = 0; n < N; ++n) {
            float cv[K];
            load_state(n, cv, sC[buf]);
            float dA[K], bb[K];
#pragma unroll
            for (int i = 0; i < K; ++i) {
                dA[i] = exp2_hw(delta[i] * ap);
                bb[i] = u[i] * bv[i];
            }
            float hl = bb[0];
#pragma unroll
            for (int i = 1; i < K; ++i) hl = __builtin_fmaf(dA[i], hl, bb[i]);
            float aa = exp2_hw(sumd * ap);
            float hend, h;
            row_scan(aa, hl, carry, hend, h);
            if (j == kRow - 1) sCarry[c * N + n] = hend;
            const int nn = (n + 1 < N) ? n + 1 : n;
            load_state(nn, bv, sB[buf]);
            ap = sA[c * N + nn];
            carry = sCarry[c * N + nn];
#pragma unroll
            for (int i = 0; i < K; ++i) {
                h = __builtin_fmaf(dA[i], h, bb[i]);
                yv[i] = __builtin_fmaf(cv[i], h, yv[i]);
            }
        }

        if (zr) {
#pragma unroll
            for (int i = 0; i < K; ++i) yv[i] *= silu(decode_raw_at<Tin, K>(zc, i));
        }
        if (live && cnt > 0) {
            Tout *yr = static_cast<Tout *>(p.y) + row + l0;
            store_y<Tout, K>(yr, cnt == K && aligned16(yr), cnt, yv);
        }
        if (ch + 1 < nchunks && stager) stage_store(buf ^ 1);
        __syncthreads();
    }

    if (p.hL && live && j == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) p.hL[(size_t(b) * dim + d) * N + n] = sCarry[c * N + n];
    }
}

template <typename Tin, typename Tout, int N>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream)
{
    constexpr int K = 16;
    ScanParams p{a.dim, a.seqlen, a.x, a.dt, a.dt_bias, a.A, a.Bm, a.Cm,
                 a.Dskip, a.z, a.h0, a.y, a.hL};
    dim3 grid((a.dim + kChannels - 1) / kChannels, a.batch);
    hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, N, K>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_n(const ScanArgs &a, hipStream_t stream)
{
    switch (a.dstate) {
    case 1: return launch_typed<Tin, Tout, 1>(a, stream);
    case 2: return launch_typed<Tin, Tout, 2>(a, stream);
    case 4: return launch_typed<Tin, Tout, 4>(a, stream);
    case 8: return launch_typed<Tin, Tout, 8>(a, stream);
    case 16: return launch_typed<Tin, Tout, 16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_fwd(const ScanArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? launch_n<bf16_t, bf16_t>(a, stream) : launch_n<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? launch_n<float, bf16_t>(a, stream) : launch_n<float, float>(a, stream);
}

}  // namespace ssm
