// scan_bld.hip -- the selective-scan forward on tensors in (batch, L, dim)
// order: time steps apart, channels contiguous, the order in which the
// reading guide's "Hardware-aware state expansion" section writes the
// (B, L, D) output back, and in which a model's input projection produces x
// and z.  Same computation as scan_fwd.hip ("Method" and "The selection
// mechanism (S6)" sections of the page "Mamba: Linear-Time Sequence Modeling
// with Selective State Spaces"):
//     Delta_t = softplus(dt_t + dt_bias[d])
//     h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t Bm[b,t,n] x_t
//     y_t     = (sum_n Cm[b,t,n] h_t[n] + Dskip[d] x_t) * silu(z_t)
// (kZoh: the exact zero-order-hold input term); only y and the final state
// reach memory.
//
// Work split.  Channels run along the lanes: a workgroup is one wave, 64
// consecutive channels of one batch row, so that every load of x, dt and z
// and every store of y at a time step is one contiguous run across the wave,
// and Bm, Cm at that step (shared by all channels) are wave-uniform.  Each
// lane keeps its channel's N states in registers and walks its piece of the
// sequence step by step: no in-chunk scan.  The sequence is cut into pieces
// (grid z) so that enough waves run at once; a piece acts on the state
// entering it as the affine map h -> exp(A sum Delta) h + e (e its end state
// from zero), and composing those maps in order is the scan's associative
// operator (the glossary's parallel associative scan).  Three launches:
//   1. bld_agg_kernel: every piece from a zero state: its end state and
//      Delta sum;
//   2. bld_combine_kernel: one thread per (batch, channel, state) composes
//      the pieces in order from h0, overwrites each piece's record with the
//      state entering it, and writes hL;
//   3. bld_main_kernel: every piece from its entering state, with the
//      readout, the gate and the output.
// No MFMA: the recurrence is not a dense contraction.
#include <algorithm>
#include <type_traits>

#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

constexpr int kLanes = 64;  // one wave: 64 consecutive channels
// Pieces per (batch, channel block): about this many waves in all.
#ifndef SSM_BLD_TARGET_WAVES
#define SSM_BLD_TARGET_WAVES 16384
#endif

struct BldParams {
    int dim, seqlen, npieces, piece_len;
    // element strides: time step, batch entry (channel / state stride 1)
    long long x_t, x_b, dt_t, dt_b, z_t, z_b, y_t, y_b, B_t, B_b, C_t, C_b;
    const float *dt_bias, *A, *Dskip, *h0;
    float *hL;
    float *rec;  // [npieces][batch][dim][N + 1]: piece maps, then entering states
    int bc_words;  // every Bm and Cm row starts on a 4-byte boundary
};

// A step's inputs are fetched as raw bits one step before they are used and
// decoded where used (the loops below alternate two such buffers), so that
// the memory latency of step t+1's loads overlaps step t's work.
template <typename T>
__device__ inline uint32_t load_bits(const T *p)
{
    if constexpr (sizeof(T) == 4) {
        return __float_as_uint(*reinterpret_cast<const float *>(p));
    } else {
        return uint32_t(p->bits);
    }
}

template <typename T>
__device__ inline float decode_bits(uint32_t w)
{
    return sizeof(T) == 4 ? __uint_as_float(w) : __uint_as_float(w << 16);
}

template <typename Tout>
__device__ inline void store_elem(Tout *p, float v)
{
    if constexpr (sizeof(Tout) == 4) {
        *reinterpret_cast<float *>(p) = v;
    } else {
        *reinterpret_cast<uint16_t *>(p) = uint16_t(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
}

// The Bm (or Cm) row of one step: N values shared by the whole wave, held as
// raw words (bf16: two states per word, fp32: one).  The address is made
// visibly wave-uniform (read from the first lane into scalar registers), and
// whole words are read as scalar loads into SGPRs once per wave instead of
// as 64-lane vector loads.  bf16 rows are read as 32-bit words only in the
// kWords instantiations, launched when every row starts on a 4-byte
// boundary (a scalar load ignores the address's two low bits); otherwise
// two 16-bit loads are packed into each word.
template <typename Tin, int N>
struct Row {
    static constexpr bool kPacked = sizeof(Tin) == 2 && N % 2 == 0;
    static constexpr int kWords = kPacked ? N / 2 : N;
    uint32_t w[kWords];
};

template <typename Tin, int N, bool kWords>
__device__ inline void row_fetch(const Tin *p, Row<Tin, N> &r)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const Tin *__restrict__ q = reinterpret_cast<const Tin *>((uint64_t(hi) << 32) | lo);
    // Whole 32-bit words are read through the constant address space: Bm and
    // Cm are never written by these kernels, and there the compiler takes
    // uniform loads as scalar loads even in a kernel that stores (the main
    // pass), so that the row and its widening stay in scalar registers
    // instead of being loaded and decoded in all 64 lanes.
    typedef const __attribute__((address_space(4))) uint32_t cword;
    if constexpr (Row<Tin, N>::kPacked) {
        if constexpr (kWords) {
            cword *u = (cword *)(reinterpret_cast<const uint32_t *>(q));
#pragma unroll
            for (int n = 0; n < N / 2; ++n) r.w[n] = u[n];
        } else {
#pragma unroll
            for (int n = 0; n < N / 2; ++n) r.w[n] = load_bits(q + 2 * n) | (load_bits(q + 2 * n + 1) << 16);
        }
    } else if constexpr (sizeof(Tin) == 4) {
        cword *u = (cword *)(reinterpret_cast<const uint32_t *>(q));
#pragma unroll
        for (int n = 0; n < N; ++n) r.w[n] = u[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) r.w[n] = load_bits(q + n);
    }
}

template <typename Tin, int N>
__device__ inline void row_decode(const Row<Tin, N> &r, float *v)
{
    if constexpr (Row<Tin, N>::kPacked) {
#pragma unroll
        for (int n = 0; n < N / 2; ++n) {
            v[2 * n] = io<bf16_t>::lo(r.w[n]);
            v[2 * n + 1] = io<bf16_t>::hi(r.w[n]);
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) v[n] = decode_bits<Tin>(r.w[n]);
    }
}

template <typename Tin, int N, bool kZoh, bool kWords>
__global__ __launch_bounds__(kLanes) void bld_agg_kernel(BldParams p, const Tin *__restrict__ x,
                                                         const Tin *__restrict__ dt,
                                                         const Tin *__restrict__ Bm)
{
    const int d = blockIdx.x * kLanes + threadIdx.x;
    const bool live = d < p.dim;
    const int dc = live ? d : p.dim - 1;
    const int b = blockIdx.y, piece = blockIdx.z;
    const int t0 = piece * p.piece_len, t1 = min(p.seqlen, t0 + p.piece_len);
    float a[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a[n] = p.A[size_t(dc) * N + n] * kLog2e;
        h[n] = 0.0f;
    }
    [[maybe_unused]] float inva[N];
    if constexpr (kZoh) {
#pragma unroll
        for (int n = 0; n < N; ++n) inva[n] = rcp_hw(a[n]) * kLog2e;
    }
    const float bias = p.dt_bias ? p.dt_bias[dc] : 0.0f;
    const Tin *xp = x + size_t(b) * size_t(p.x_b) + size_t(t0) * size_t(p.x_t) + dc;
    const Tin *dp = dt + size_t(b) * size_t(p.dt_b) + size_t(t0) * size_t(p.dt_t) + dc;
    const Tin *bp = Bm + size_t(b) * size_t(p.B_b) + size_t(t0) * size_t(p.B_t);
    float sumd = 0.0f;
    struct In {
        uint32_t x, dt;
        Row<Tin, N> b;
    };
    auto fetch = [&](In &in) {  // the next step's inputs; advances the pointers
        in.x = load_bits(xp);
        in.dt = load_bits(dp);
        row_fetch<Tin, N, kWords>(bp, in.b);
        xp += p.x_t;
        dp += p.dt_t;
        bp += p.B_t;
    };
    auto step = [&](const In &in) {
        const float xv = decode_bits<Tin>(in.x), delta = softplus(decode_bits<Tin>(in.dt) + bias);
        float bn[N];
        row_decode<Tin, N>(in.b, bn);
        const float u = delta * xv;
        [[maybe_unused]] const float invd = kZoh ? rcp_hw(delta) : 0.0f;
        sumd += delta;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float s = delta * a[n];
            const float e = exp2_hw(s);
            float bb = u * bn[n];
            if constexpr (kZoh) bb *= phi_zoh(s * kLn2, e, invd * inva[n]);
            h[n] = __builtin_fmaf(e, h[n], bb);
        }
    };
    In i0, i1;
    int t = t0;
    if (t < t1) fetch(i0);
    for (; t + 1 < t1; t += 2) {
        fetch(i1);
        step(i0);
        if (t + 2 < t1) fetch(i0);
        step(i1);
    }
    if (t < t1) step(i0);
    if (live) {
        float *r = p.rec + ((size_t(piece) * gridDim.y + b) * p.dim + d) * (N + 1);
#pragma unroll
        for (int n = 0; n < N; ++n) r[n] = h[n];
        r[N] = sumd;
    }
}

// One thread per (batch, channel, state): the state entering every piece,
// written over that piece's map (read first, by the same thread), and hL.
template <int N>
__global__ __launch_bounds__(256) void bld_combine_kernel(BldParams p, int batch)
{
    const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
    const size_t rows = size_t(batch) * p.dim;
    if (i >= rows * N) return;
    const int n = int(i % N);
    const size_t row = i / N;  // b * dim + d
    const int d = int(row % size_t(p.dim));
    const float a = p.A[size_t(d) * N + n] * kLog2e;
    float h = p.h0 ? p.h0[row * N + n] : 0.0f;
    // Pieces in groups of kG: the group's records are all loaded before the
    // first is composed, so that the loads' latency is paid once per group
    // rather than once per piece (each piece's entering state overwrites its
    // own record's e, already in registers).
    constexpr int kG = 8;
    const size_t pstride = rows * (N + 1);
    float *r0 = p.rec + row * (N + 1);
    int k = 0;
    for (; k + kG <= p.npieces; k += kG) {
        float sd[kG], e[kG];
#pragma unroll
        for (int j = 0; j < kG; ++j) {
            const float *r = r0 + size_t(k + j) * pstride;
            sd[j] = r[N];
            e[j] = r[n];
        }
#pragma unroll
        for (int j = 0; j < kG; ++j) {
            r0[size_t(k + j) * pstride + n] = h;
            h = __builtin_fmaf(exp2_hw(a * sd[j]), h, e[j]);
        }
    }
    for (; k < p.npieces; ++k) {
        float *r = r0 + size_t(k) * pstride;
        const float sd = r[N], e = r[n];
        r[n] = h;
        h = __builtin_fmaf(exp2_hw(a * sd), h, e);
    }
    if (p.hL) p.hL[row * N + n] = h;
}

template <typename Tin, typename Tout, int N, bool kZoh, bool kWords>
__global__ __launch_bounds__(kLanes) void bld_main_kernel(
    BldParams p, const Tin *__restrict__ x, const Tin *__restrict__ dt, const Tin *__restrict__ z,
    const Tin *__restrict__ Bm, const Tin *__restrict__ Cm, Tout *__restrict__ y)
{
    const int d = blockIdx.x * kLanes + threadIdx.x;
    const bool live = d < p.dim;
    const int dc = live ? d : p.dim - 1;
    const int b = blockIdx.y, piece = blockIdx.z;
    const int t0 = piece * p.piece_len, t1 = min(p.seqlen, t0 + p.piece_len);
    const float *r = p.rec + ((size_t(piece) * gridDim.y + b) * p.dim + dc) * (N + 1);
    float a[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a[n] = p.A[size_t(dc) * N + n] * kLog2e;
        h[n] = r[n];
    }
    [[maybe_unused]] float inva[N];
    if constexpr (kZoh) {
#pragma unroll
        for (int n = 0; n < N; ++n) inva[n] = rcp_hw(a[n]) * kLog2e;
    }
    const float bias = p.dt_bias ? p.dt_bias[dc] : 0.0f;
    const float skip = p.Dskip ? p.Dskip[dc] : 0.0f;
    const Tin *xp = x + size_t(b) * size_t(p.x_b) + size_t(t0) * size_t(p.x_t) + dc;
    const Tin *dp = dt + size_t(b) * size_t(p.dt_b) + size_t(t0) * size_t(p.dt_t) + dc;
    const Tin *zp = z ? z + size_t(b) * size_t(p.z_b) + size_t(t0) * size_t(p.z_t) + dc : nullptr;
    Tout *yp = y + size_t(b) * size_t(p.y_b) + size_t(t0) * size_t(p.y_t) + dc;
    const Tin *bp = Bm + size_t(b) * size_t(p.B_b) + size_t(t0) * size_t(p.B_t);
    const Tin *cp = Cm + size_t(b) * size_t(p.C_b) + size_t(t0) * size_t(p.C_t);
    struct In {
        uint32_t x, dt, z;
        Row<Tin, N> b, c;
    };
    auto fetch = [&](In &in) {  // the next step's inputs; advances the pointers
        in.x = load_bits(xp);
        in.dt = load_bits(dp);
        in.z = zp ? load_bits(zp) : 0u;
        row_fetch<Tin, N, kWords>(bp, in.b);
        row_fetch<Tin, N, kWords>(cp, in.c);
        xp += p.x_t;
        dp += p.dt_t;
        if (zp) zp += p.z_t;
        bp += p.B_t;
        cp += p.C_t;
    };
    auto step = [&](const In &in) {
        const float xv = decode_bits<Tin>(in.x), delta = softplus(decode_bits<Tin>(in.dt) + bias);
        float bn[N], cn[N];
        row_decode<Tin, N>(in.b, bn);
        row_decode<Tin, N>(in.c, cn);
        const float u = delta * xv;
        [[maybe_unused]] const float invd = kZoh ? rcp_hw(delta) : 0.0f;
        float yv = skip * xv;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float s = delta * a[n];
            const float e = exp2_hw(s);
            float bb = u * bn[n];
            if constexpr (kZoh) bb *= phi_zoh(s * kLn2, e, invd * inva[n]);
            h[n] = __builtin_fmaf(e, h[n], bb);
            yv = __builtin_fmaf(cn[n], h[n], yv);
        }
        if (z) yv *= silu(decode_bits<Tin>(in.z));
        if (live) store_elem(yp, yv);
        yp += p.y_t;
    };
    In i0, i1;
    int t = t0;
    if (t < t1) fetch(i0);
    for (; t + 1 < t1; t += 2) {
        fetch(i1);
        step(i0);
        if (t + 2 < t1) fetch(i0);
        step(i1);
    }
    if (t < t1) step(i0);
}

// Pieces: about 16384 waves in all (four rounds at four per SIMD: the more
// waves in flight, the better the per-step loads' latency is hidden, and
// extra pieces cost only their composition), at least 64 steps each.
BldSplit bld_split_impl(int batch, int dim, int seqlen)
{
    const long long waves = (long long)batch * ((dim + kLanes - 1) / kLanes);
    long long np = (SSM_BLD_TARGET_WAVES + waves - 1) / waves;
    np = std::max(1LL, std::min<long long>(np, seqlen / 64));
    np = std::min<long long>(np, 65535);
    BldSplit s;
    s.piece_len = int((seqlen + np - 1) / np);
    s.npieces = (seqlen + s.piece_len - 1) / s.piece_len;
    return s;
}

template <typename Tin, typename Tout, int N, bool kZoh>
hipError_t launch_typed(const BldArgs &a, hipStream_t stream)
{
    const BldSplit sp = bld_split_impl(a.batch, a.dim, a.seqlen);
    BldParams p{a.dim, a.seqlen, sp.npieces, sp.piece_len,
                a.x_t, a.x_b, a.dt_t, a.dt_b, a.z_t, a.z_b, a.y_t, a.y_b,
                a.B_t, a.B_b, a.C_t, a.C_b, a.dt_bias, a.A, a.Dskip, a.h0, a.hL, a.workspace, 0};
    // bf16 Bm / Cm rows can be read as words when every row is word-aligned
    auto words = [](const void *base, long long st, long long sb) {
        return (reinterpret_cast<uintptr_t>(base) & 3) == 0 && (st * 2) % 4 == 0 &&
               (sb * 2) % 4 == 0;
    };
    p.bc_words = words(a.Bm, a.B_t, a.B_b) && words(a.Cm, a.C_t, a.C_b);
    const dim3 grid((unsigned(a.dim) + kLanes - 1) / kLanes, a.batch, sp.npieces);
    const size_t threads = size_t(a.batch) * a.dim * N;
    if (log_enabled())
        log_line("scan_fwd_bld: %d pieces of %d steps: bld_agg_kernel<in %s, N %d, zoh %d>, "
                 "bld_combine_kernel, bld_main_kernel<out %s>, grid (%u, %u, %u) x %d threads",
                 sp.npieces, sp.piece_len, type_tag<Tin>(), N, int(kZoh), type_tag<Tout>(), grid.x,
                 grid.y, grid.z, kLanes);
    const Tin *x = static_cast<const Tin *>(a.x), *dt = static_cast<const Tin *>(a.dt);
    const Tin *Bm = static_cast<const Tin *>(a.Bm), *Cm = static_cast<const Tin *>(a.Cm);
    // bf16 rows of two states per word: a separate instantiation for word-aligned rows, so
    // that the row loads are scalar loads with no per-lane alternative in the loop
    auto launch = [&](auto words) -> hipError_t {
        constexpr bool kW = decltype(words)::value;
        hipLaunchKernelGGL((bld_agg_kernel<Tin, N, kZoh, kW>), grid, dim3(kLanes), 0, stream, p, x, dt,
                           Bm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bld_combine_kernel<N>), dim3(unsigned((threads + 255) / 256)), dim3(256), 0,
                           stream, p, a.batch);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bld_main_kernel<Tin, Tout, N, kZoh, kW>), grid, dim3(kLanes), 0, stream, p,
                           x, dt, static_cast<const Tin *>(a.z), Bm, Cm, static_cast<Tout *>(a.y));
        return hipGetLastError();
    };
    if (Row<Tin, N>::kPacked && p.bc_words) return launch(std::true_type{});
    return launch(std::false_type{});
}

template <typename Tin, typename Tout, bool kZoh>
hipError_t launch_n(const BldArgs &a, hipStream_t stream)
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
hipError_t launch_mode(const BldArgs &a, hipStream_t stream)
{
    return a.zoh ? launch_n<Tin, Tout, true>(a, stream) : launch_n<Tin, Tout, false>(a, stream);
}

}  // namespace

BldSplit bld_split(int batch, int dim, int seqlen) { return bld_split_impl(batch, dim, seqlen); }

size_t scan_bld_workspace_bytes(int batch, int dim, int seqlen, int dstate)
{
    const BldSplit sp = bld_split_impl(batch, dim, seqlen);
    return size_t(sp.npieces) * size_t(batch) * size_t(dim) * size_t(dstate + 1) * sizeof(float);
}

hipError_t launch_scan_bld(const BldArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? launch_mode<bf16_t, bf16_t>(a, stream)
                          : launch_mode<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? launch_mode<float, bf16_t>(a, stream) : launch_mode<float, float>(a, stream);
}

}  // namespace ssm
