// conv1d.hip -- causal depthwise 1-D convolution that feeds the selective
// scan, and its single-token decode step, for gfx950.
//
// The Mamba block runs a short 1-D convolution over the sequence before the
// selective SSM (glossary entry "Mamba Block" of the page "Mamba: Linear-Time
// Sequence Modeling with Selective State Spaces"; d_conv = 4 in the
// basic-model example of the page "Mamba选择性状态空间机制：效率提升10倍的核心突破"),
// and the inference cache keeps
// its convolutional state beside the SSM state ("everything-about-mamba-paper").
// Per (batch b, channel d), with the W-1 inputs before t = 0 taken from the
// conv state (oldest first) or zero:
//     y[t] = act(bias[d] + sum_k weight[d][k] * x[t - (W-1) + k])
// so weight[d][W-1] meets the current input; act is silu or the identity.
//
// The forward pass reads each input once and writes each output once: it is
// bound by HBM bandwidth, not arithmetic (W fma + one silu per output).  A
// lane owns 16 consecutive outputs of one row (two 16-byte vectors of bf16
// in flight per lane; 8 measured 5 % slower, 32 much slower); consecutive
// lanes own consecutive runs of the same row, so a wave reads and writes
// contiguous 2 KB (bf16) stretches with 16-byte vector accesses.  The W-1 inputs before a
// run are the previous lane's last inputs (a lane shuffle, so every input is
// read from memory once), the conv state for a row's first run, or, for lane 0
// of a wave, W-1 element loads.
// The first run's lane also writes the row's final conv state, after reading
// the initial one, so the two may be the same buffer.
#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

#ifndef SSM_CONV_RUN
#define SSM_CONV_RUN 16
#endif
constexpr int kRun = SSM_CONV_RUN;  // outputs per lane (a multiple of 8)
static_assert(kRun % 8 == 0, "runs are whole 16-byte vectors of bf16 and fp32");
constexpr int kConvThreads = 256;

struct ConvParams {
    int dim, seqlen, runs_per_row;
    unsigned div_mul, div_shift;  // g / runs_per_row == (umulhi(g, mul) + g) >> shift
    unsigned dim_mul, dim_shift;  // row / dim likewise
    long long total_runs;
    // element strides (time contiguous): channel rows and batch entries
    long long x_row, x_b, y_row, y_b;
    const void *x;
    const float *weight, *bias, *state0;
    void *y;
    float *stateL;
};

// Division by a fixed divisor 1 <= d < 2^31 through one high multiply
// (round-up reciprocal: m = floor(2^32 (2^s - d) / d) + 1 with 2^s >= d),
// exact for every 32-bit numerator.
struct MagicDiv {
    unsigned mul, shift;
};

MagicDiv magic_div(unsigned d)
{
    unsigned s = 0;
    while ((1ull << s) < d) ++s;
    const unsigned long long m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return {unsigned(m), s};
}

__device__ inline unsigned div_magic(unsigned n, unsigned mul, unsigned shift)
{
    const unsigned t = __umulhi(n, mul);
    return unsigned((static_cast<unsigned long long>(t) + n) >> shift);
}

template <int W>
__device__ inline void load_taps(const float *w, float *taps)
{
#pragma unroll
    for (int k = 0; k < W; ++k) taps[k] = w[k];
}

template <typename Tout>
__device__ inline void store_run(Tout *p, bool vec, int count, const float *v);

template <>
__device__ inline void store_run<float>(float *p, bool vec, int count, const float *v)
{
    if (vec) {
        f32x4 *q = reinterpret_cast<f32x4 *>(p);
#pragma unroll
        for (int i = 0; i < kRun / 4; ++i)
            q[i] = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < kRun; ++i)
            if (i < count) p[i] = v[i];
    }
}

template <>
__device__ inline void store_run<bf16_t>(bf16_t *p, bool vec, int count, const float *v)
{
    if (vec) {
        u32x4 *q = reinterpret_cast<u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < kRun / 8; ++i) {
            const float *w = v + 8 * i;
            q[i] = u32x4{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]),
                         pack_bf16x2(w[4], w[5]), pack_bf16x2(w[6], w[7])};
        }
    } else {
#pragma unroll
        for (int i = 0; i < kRun; ++i)
            if (i < count) p[i].bits = uint16_t(pack_bf16x2(v[i], 0.0f) & 0xffffu);
    }
}

// vec_in / vec_out: every run of every row starts on a 16-byte boundary of x
// (resp. y), decided on the host from the base addresses and seqlen.
template <typename Tin, typename Tout, int W, bool kWide>
__global__ void __launch_bounds__(kConvThreads)
conv1d_fwd_kernel(ConvParams p, bool vec_in, bool vec_out, bool act)
{
    constexpr int H = W - 1;
    const long long g = (long long)blockIdx.x * kConvThreads + threadIdx.x;
    const bool live = g < p.total_runs;
    long long row, bi;  // row = bi * dim + d
    int j;
    if constexpr (kWide) {
        row = g / p.runs_per_row;
        j = int(g - row * p.runs_per_row);
        bi = row / p.dim;
    } else {
        const unsigned q = div_magic(unsigned(g), p.div_mul, p.div_shift);
        row = q;
        j = int(unsigned(g) - q * unsigned(p.runs_per_row));
        bi = div_magic(q, p.dim_mul, p.dim_shift);
    }
    const int d = int(row - bi * p.dim);
    const int L = p.seqlen;
    const int t0 = j * kRun;
    const int count = live ? min(kRun, L - t0) : 0;

    const Tin *xr = static_cast<const Tin *>(p.x) + bi * p.x_b + d * p.x_row;
    float e[H + kRun];  // e[H + i] = x[t0 + i]; e[0..H) the inputs before the run
    if (live) {
        load_run<Tin, kRun>(xr + t0, vec_in && count == kRun, count, e + H);
    } else {
#pragma unroll
        for (int i = 0; i < H + kRun; ++i) e[i] = 0.0f;
    }
    // The H inputs before the run are the previous lane's last H inputs when
    // that lane holds the previous run of the same row (j > 0, not lane 0).
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < H; ++k) e[k] = __shfl_up(e[kRun + k], 1, 64);
    if (!live) return;
    if (j == 0) {
#pragma unroll
        for (int k = 0; k < H; ++k) e[k] = p.state0 ? p.state0[row * H + k] : 0.0f;
    } else if (lane == 0) {
#pragma unroll
        for (int k = 0; k < H; ++k) e[k] = io<Tin>::load1(xr + t0 - H + k);
    }
    float taps[W];
    load_taps<W>(p.weight + (size_t)d * W, taps);
    const float b = p.bias ? p.bias[d] : 0.0f;
    float out[kRun];
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
        float s = b;
#pragma unroll
        for (int k = 0; k < W; ++k) s = __builtin_fmaf(taps[k], e[i + k], s);
        out[i] = act ? silu(s) : s;
    }
    store_run<Tout>(static_cast<Tout *>(p.y) + bi * p.y_b + d * p.y_row + t0,
                    vec_out && count == kRun, count, out);

    if (j == 0 && p.stateL) {
        // Final state = the last H entries of (state0, x).  This lane already
        // holds state0 in e[0..H); entries inside x are read from memory.
        float fin[H > 0 ? H : 1];
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const int idx = L - H + k;  // position in x; < 0 means inside state0
            fin[k] = idx >= 0 ? io<Tin>::load1(xr + idx) : e[idx + H];
        }
#pragma unroll
        for (int k = 0; k < H; ++k) p.stateL[row * H + k] = fin[k];
    }
}

struct ConvUpdateParams {
    int batch, dim;
    float *state;
    const void *x;
    const float *weight, *bias;
    void *y;
    long long x_b, y_b;  // batch strides in elements
};

// One lane per (batch, channel): y = act(bias + sum_k w[k] e[k]) over
// e = (state, x), then state <- the last W-1 entries of e, in place.
template <typename Tin, typename Tout, int W>
__global__ void __launch_bounds__(kConvThreads)
conv1d_update_kernel(ConvUpdateParams p, bool act)
{
    constexpr int H = W - 1;
    const long long row = (long long)blockIdx.x * kConvThreads + threadIdx.x;
    if (row >= (long long)p.batch * p.dim) return;
    const long long bi = row / p.dim;
    const int d = int(row - bi * p.dim);
    float e[W];
#pragma unroll
    for (int k = 0; k < H; ++k) e[k] = p.state[row * H + k];
    e[H] = io<Tin>::load1(static_cast<const Tin *>(p.x) + bi * p.x_b + d);
    float taps[W];
    load_taps<W>(p.weight + (size_t)d * W, taps);
    float s = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) s = __builtin_fmaf(taps[k], e[k], s);
    const float v = act ? silu(s) : s;
    const long long yi = bi * p.y_b + d;
    if constexpr (sizeof(Tout) == 4) {
        static_cast<float *>(p.y)[yi] = v;
    } else {
        static_cast<bf16_t *>(p.y)[yi].bits = uint16_t(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
#pragma unroll
    for (int k = 0; k < H; ++k) p.state[row * H + k] = e[k + 1];
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

template <typename Tin, typename Tout, int W>
hipError_t launch_conv_typed(const ConvArgs &a, hipStream_t stream)
{
    ConvParams p;
    p.dim = a.dim;
    p.seqlen = a.seqlen;
    p.runs_per_row = (a.seqlen + kRun - 1) / kRun;
    p.total_runs = (long long)a.batch * a.dim * p.runs_per_row;
    p.x = a.x;
    p.weight = a.weight;
    p.bias = a.bias;
    p.state0 = a.state0;
    p.y = a.y;
    p.stateL = a.stateL;
    p.x_row = a.x_row;
    p.x_b = a.x_b;
    p.y_row = a.y_row;
    p.y_b = a.y_b;
    const MagicDiv md = magic_div(unsigned(a.dim));
    p.dim_mul = md.mul;
    p.dim_shift = md.shift;
    // Every run starts at element b * batch stride + d * row stride + 8 j;
    // 16-byte vectors need each term times the element size to be a multiple
    // of 16 on a 16-byte base.
    auto vec16 = [](const void *base, size_t esize, long long row, long long bs) {
        return aligned16(base) && (size_t(row) * esize) % 16 == 0 && (size_t(bs) * esize) % 16 == 0 &&
               (kRun * esize) % 16 == 0;
    };
    const bool vec_in = vec16(a.x, sizeof(Tin), a.x_row, a.x_b);
    const bool vec_out = vec16(a.y, sizeof(Tout), a.y_row, a.y_b);
    const long long blocks = (p.total_runs + kConvThreads - 1) / kConvThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (log_enabled())
        log_line("conv1d_fwd: conv1d_fwd_kernel<in %s, out %s, W %d>, %lld runs of %d outputs, "
                 "%lld workgroups x %d threads, %s-bit row index, vector in %d out %d",
                 type_tag<Tin>(), type_tag<Tout>(), W, (long long)p.total_runs, kRun, blocks,
                 kConvThreads, p.total_runs + kConvThreads <= (1ll << 32) ? "32" : "64",
                 int(vec_in), int(vec_out));
    if (p.total_runs + kConvThreads <= (1ll << 32)) {
        const MagicDiv m = magic_div(unsigned(p.runs_per_row));
        p.div_mul = m.mul;
        p.div_shift = m.shift;
        hipLaunchKernelGGL((conv1d_fwd_kernel<Tin, Tout, W, false>), dim3(unsigned(blocks)),
                           dim3(kConvThreads), 0, stream, p, vec_in, vec_out, a.silu != 0);
    } else {
        hipLaunchKernelGGL((conv1d_fwd_kernel<Tin, Tout, W, true>), dim3(unsigned(blocks)),
                           dim3(kConvThreads), 0, stream, p, vec_in, vec_out, a.silu != 0);
    }
    return hipGetLastError();
}

template <typename Tin, typename Tout, int W>
hipError_t launch_update_typed(const ConvUpdateArgs &a, hipStream_t stream)
{
    ConvUpdateParams p{a.batch, a.dim, a.state, a.x, a.weight, a.bias, a.y, a.x_b, a.y_b};
    const long long rows = (long long)a.batch * a.dim;
    const long long blocks = (rows + kConvThreads - 1) / kConvThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (log_enabled())
        log_line("conv1d_update: conv1d_update_kernel<in %s, out %s, W %d>, %lld workgroups x %d "
                 "threads", type_tag<Tin>(), type_tag<Tout>(), W, blocks, kConvThreads);
    hipLaunchKernelGGL((conv1d_update_kernel<Tin, Tout, W>), dim3(unsigned(blocks)),
                       dim3(kConvThreads), 0, stream, p, a.silu != 0);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t conv_width(const ConvArgs &a, hipStream_t s)
{
    switch (a.width) {
    case 2: return launch_conv_typed<Tin, Tout, 2>(a, s);
    case 3: return launch_conv_typed<Tin, Tout, 3>(a, s);
    case 4: return launch_conv_typed<Tin, Tout, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tin, typename Tout>
hipError_t update_width(const ConvUpdateArgs &a, hipStream_t s)
{
    switch (a.width) {
    case 2: return launch_update_typed<Tin, Tout, 2>(a, s);
    case 3: return launch_update_typed<Tin, Tout, 3>(a, s);
    case 4: return launch_update_typed<Tin, Tout, 4>(a, s);
    }
    return hipErrorInvalidValue;
}


// ---------------------------------------------------------------- (batch, L, dim) order
// The same convolution on x and y whose channels are contiguous and whose time
// steps are `*_t` elements apart (the order a model's input projection
// produces).  A lane owns V consecutive channels (V = 4 when every access of
// the call can be one 4-element vector, else 1) and walks a piece of
// consecutive steps, keeping the W-1 previous inputs of its channels in
// registers; a wave reads and writes 64 V consecutive channels of one step per
// access.  Pieces are walked by separate workgroups: each re-reads the W-1
// inputs before its first step (the first piece takes them from the conv
// state).  The first piece's lanes also write the final conv state, after
// reading the initial one, so the two may be the same buffer.
struct ConvBldParams {
    int dim, seqlen, piece, cblocks;
    long long x_t, x_b, y_t, y_b;
    const void *x;
    const float *weight, *bias, *state0;
    void *y;
    float *stateL;
};

template <typename T, int V>
__device__ inline void bld_load(const T *p, float *v)
{
    if constexpr (V == 1) {
        v[0] = io<T>::load1(p);
    } else if constexpr (sizeof(T) == 4) {
        const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    } else {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        v[0] = io<bf16_t>::lo(w.x); v[1] = io<bf16_t>::hi(w.x);
        v[2] = io<bf16_t>::lo(w.y); v[3] = io<bf16_t>::hi(w.y);
    }
}

template <typename T, int V>
__device__ inline void bld_store(T *p, const float *v)
{
    if constexpr (sizeof(T) == 4) {
        if constexpr (V == 1) {
            *reinterpret_cast<float *>(p) = v[0];
        } else {
            *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
        }
    } else {
        if constexpr (V == 1) {
            reinterpret_cast<bf16_t *>(p)->bits = uint16_t(pack_bf16x2(v[0], 0.0f) & 0xffffu);
        } else {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
}

template <typename Tin, typename Tout, int W, int V>
__global__ void __launch_bounds__(kConvThreads)
conv1d_bld_kernel(ConvBldParams p, bool act)
{
    constexpr int H = W - 1;
    // steps whose loads are issued before the first is used: at the 2.8B layer
    // (bf16 in and out) 1 / 2 / 4 / 8 steps took 40.3 / 34.5 / 36.7 / 38.5 us
    constexpr int U = 2;
    const int cb = int(blockIdx.x % unsigned(p.cblocks));
    const int b = int(blockIdx.x / unsigned(p.cblocks));
    const int d0 = (cb * kConvThreads + int(threadIdx.x)) * V;  // first channel of the lane
    if (d0 >= p.dim) return;  // dim is a multiple of V: the lane's channels are all live
    const int t0 = int(blockIdx.y) * p.piece;
    const int t1 = min(p.seqlen, t0 + p.piece);
    const Tin *xb = static_cast<const Tin *>(p.x) + size_t(b) * size_t(p.x_b) + d0;
    Tout *yb = static_cast<Tout *>(p.y) + size_t(b) * size_t(p.y_b) + d0;
    const size_t row = size_t(b) * size_t(p.dim) + size_t(d0);  // conv-state row of channel d0

    float w[W][V], bias[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int k = 0; k < W; ++k) w[k][v] = p.weight[size_t(d0 + v) * W + k];
        bias[v] = p.bias ? p.bias[d0 + v] : 0.0f;
    }
    // h[k]: the input at step t - H + k before the step t being computed
    float h[H > 0 ? H : 1][V];
    if (t0 == 0) {
#pragma unroll
        for (int k = 0; k < H; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v) h[k][v] = p.state0 ? p.state0[(row + v) * H + k] : 0.0f;
        if (p.stateL) {
            // final state: the last H entries of (state0, x)
            float fin[H > 0 ? H : 1][V];
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int idx = p.seqlen - H + k;  // < 0: inside state0
                if (idx >= 0) {
                    bld_load<Tin, V>(xb + size_t(idx) * size_t(p.x_t), fin[k]);
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v) fin[k][v] = h[idx + H][v];
                }
            }
#pragma unroll
            for (int k = 0; k < H; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v) p.stateL[(row + v) * H + k] = fin[k][v];
        }
    } else {
#pragma unroll
        for (int k = 0; k < H; ++k) bld_load<Tin, V>(xb + size_t(t0 - H + k) * size_t(p.x_t), h[k]);
    }

    const Tin *xp = xb + size_t(t0) * size_t(p.x_t);
    Tout *yp = yb + size_t(t0) * size_t(p.y_t);
    for (int t = t0; t < t1; t += U) {
        float xv[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t + u < t1) {
                bld_load<Tin, V>(xp + size_t(u) * size_t(p.x_t), xv[u]);
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) xv[u][v] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t + u >= t1) break;
            float out[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                // the [batch][dim][L] kernel's order: bias, then the oldest input first
                float s = bias[v];
#pragma unroll
                for (int k = 0; k < H; ++k) s = __builtin_fmaf(w[k][v], h[k][v], s);
                s = __builtin_fmaf(w[H][v], xv[u][v], s);
                out[v] = act ? silu(s) : s;
            }
            bld_store<Tout, V>(yp + size_t(u) * size_t(p.y_t), out);
#pragma unroll
            for (int k = 0; k + 1 < H; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v) h[k][v] = h[k + 1][v];
#pragma unroll
            for (int v = 0; v < V; ++v) h[H - 1][v] = xv[u][v];
        }
        xp += size_t(U) * size_t(p.x_t);
        yp += size_t(U) * size_t(p.y_t);
    }
}

template <typename Tin, typename Tout, int W>
hipError_t launch_bld_typed(const ConvBldArgs &a, hipStream_t stream)
{
    // 4-channel vectors when every lane's every access starts on a multiple
    // of 4 elements of an aligned base
    auto vec4 = [](const void *base, size_t esize, long long st, long long bs) {
        return (reinterpret_cast<uintptr_t>(base) % (4 * esize)) == 0 && st % 4 == 0 && bs % 4 == 0;
    };
    const bool v4 = a.dim % 4 == 0 && vec4(a.x, sizeof(Tin), a.x_t, a.x_b) &&
                    vec4(a.y, sizeof(Tout), a.y_t, a.y_b);
    const int V = v4 ? 4 : 1;
    ConvBldParams p;
    p.dim = a.dim;
    p.seqlen = a.seqlen;
    p.cblocks = int((a.dim + kConvThreads * V - 1) / (kConvThreads * V));
    p.x_t = a.x_t;
    p.x_b = a.x_b;
    p.y_t = a.y_t;
    p.y_b = a.y_b;
    p.x = a.x;
    p.weight = a.weight;
    p.bias = a.bias;
    p.state0 = a.state0;
    p.y = a.y;
    p.stateL = a.stateL;
    // Pieces of 64 steps, halved (to 16 at least) while the launch has fewer
    // than ~4 waves per SIMD; at most 65535 pieces.
    const long long waves_per_piece = (long long)a.batch * p.cblocks * (kConvThreads / 64);
    long long piece = 64;
    while (piece > 16 && waves_per_piece * ((a.seqlen + piece - 1) / piece) < 4096) piece /= 2;
    if ((a.seqlen + piece - 1) / piece > 65535) piece = (a.seqlen + 65534) / 65535;
    p.piece = int(piece);
    const long long npieces = (a.seqlen + piece - 1) / piece;
    const long long gx = (long long)a.batch * p.cblocks;
    if (gx > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (log_enabled())
        log_line("conv1d_fwd_bld: conv1d_bld_kernel<in %s, out %s, W %d, channels per lane %d>, "
                 "grid (%lld, %lld) x %d threads, pieces of %lld steps",
                 type_tag<Tin>(), type_tag<Tout>(), W, V, gx, npieces, kConvThreads, piece);
    const dim3 grid{unsigned(gx), unsigned(npieces), 1u};
    if (v4) {
        hipLaunchKernelGGL((conv1d_bld_kernel<Tin, Tout, W, 4>), grid, dim3(kConvThreads), 0,
                           stream, p, a.silu != 0);
    } else {
        hipLaunchKernelGGL((conv1d_bld_kernel<Tin, Tout, W, 1>), grid, dim3(kConvThreads), 0,
                           stream, p, a.silu != 0);
    }
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t bld_width(const ConvBldArgs &a, hipStream_t s)
{
    switch (a.width) {
    case 2: return launch_bld_typed<Tin, Tout, 2>(a, s);
    case 3: return launch_bld_typed<Tin, Tout, 3>(a, s);
    case 4: return launch_bld_typed<Tin, Tout, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? conv_width<bf16_t, bf16_t>(a, stream) : conv_width<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? conv_width<float, bf16_t>(a, stream) : conv_width<float, float>(a, stream);
}

hipError_t launch_conv1d_update(const ConvUpdateArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? update_width<bf16_t, bf16_t>(a, stream)
                          : update_width<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? update_width<float, bf16_t>(a, stream) : update_width<float, float>(a, stream);
}

hipError_t launch_conv1d_bld(const ConvBldArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? bld_width<bf16_t, bf16_t>(a, stream) : bld_width<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? bld_width<float, bf16_t>(a, stream) : bld_width<float, float>(a, stream);
}

}  // namespace ssm
