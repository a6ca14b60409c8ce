// scan_fwd.hip -- fused selective-scan forward pass for gfx950.
//
// Computes, per (batch b, channel d), over t = 0..L-1
// ("Method" and "The selection mechanism (S6)" sections of the page
// "Mamba: Linear-Time Sequence Modeling with Selective State Spaces"):
//     Delta_t = softplus(dt_t + dt_bias[d])
//     h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t Bm[b,n,t] x_t
//     y_t     = (sum_n Cm[b,n,t] h_t[n] + Dskip[d] x_t) * silu(z_t)
// (kZoh: the input term is the exact zero-order-hold B-bar of "Method",
// phi(Delta_t A[d,n]) Delta_t Bm[b,n,t] x_t with phi(x) = (e^x - 1) / x.)
// with the state expansion kept on chip ("Hardware-aware state expansion"):
// only y and the final state are written to HBM.
//
// Work split.  A workgroup of kWaves waves owns one batch row and 4 kWaves
// channels.  Each 16-lane DPP row of a wave owns one channel; lane j of the
// row owns the K consecutive timesteps [l0 + jK, l0 + jK + K) of a chunk of
// 16K timesteps.  K = 8 keeps the kernel at <= 128 VGPRs and ~36 KB of LDS
// per 4-wave workgroup, i.e. four waves per SIMD; a single wave issues VALU
// work far below the SIMD's rate, so the scan needs the occupancy more than
// it needs longer per-lane runs.
// The workgroup walks the sequence chunk by chunk.  For each state n:
//   1. each lane folds its K steps into one affine map h -> a h + b
//      (a = exp2(A' sum Delta), b by a K-step fma chain),
//   2. a 4-level DPP row scan composes the 16 maps (the associative scan of
//      "Hardware-aware state expansion"; the chunking follows the chunked
//      computation of the page "Mamba选择性状态空间机制：效率提升10倍的核心突破"),
//   3. each lane applies its prefix to the carry entering the chunk and
//      replays its K steps, accumulating C_t h_t into y_t,
//   4. the row's last lane publishes the carry for the next chunk in LDS.
// Bm and Cm chunks (shared by every channel of the batch row) are staged once
// per workgroup into LDS as fp32, double-buffered, one barrier per chunk.
// No MFMA: the recurrence is not a dense contraction.
#include <algorithm>

#include "scan_common.hpp"
#include "ssm_device.hpp"
#include "ssm_launch.hpp"

namespace ssm {
namespace {

// Tuning constants (overridable at build time for sweeps).
#ifndef SSM_SCAN_WAVES
#define SSM_SCAN_WAVES 4
#endif
#ifndef SSM_SCAN_K
#define SSM_SCAN_K 8
#endif
#ifndef SSM_SCAN_PAIRS
#define SSM_SCAN_PAIRS 1
#endif
#ifndef SSM_SCAN_MINW_BF16
#define SSM_SCAN_MINW_BF16 4
#endif
#ifndef SSM_SCAN_MINW_F32
#define SSM_SCAN_MINW_F32 4
#endif
constexpr int kRow = 16;                    // lanes per channel (one DPP row)
constexpr int kWaves = SSM_SCAN_WAVES;      // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kChannels = kThreads / kRow;  // channels per workgroup
constexpr int kK = SSM_SCAN_K;              // consecutive timesteps per lane
// Sequence split (see scan_fwd_split): used when the batch rows and channel
// blocks give fewer than SSM_SPLIT_BELOW_WGS workgroups; aims at
// kSplitTargetWgs workgroups (ssm_launch.hpp) with segments of at least
// SSM_SPLIT_MIN_STEPS steps.  The aggregate pass costs about 0.6 of a main
// pass, so a split pays where the unsplit launch runs the chip at under
// about half its rate: measured, fewer than ~300 workgroups (a 2x to 4x gain
// at 48 to 128 workgroups, a loss at 320 with two segments).  Many segments
// (~64 workgroups per CU) keep the last wave's tail short: at batch 1, 1536
// channels and 2^20 steps, targets of 4096 / 16384 / 32768 workgroups
// measured 14.61 / 14.15 / 15.75 ms per forward call, and the backward call
// 45.5 ms at 4096 against 44.5 ms at 16384.
#ifndef SSM_SPLIT_BELOW_WGS
#define SSM_SPLIT_BELOW_WGS 256
#endif
#ifndef SSM_SPLIT_MIN_STEPS
#define SSM_SPLIT_MIN_STEPS 1024
#endif
constexpr int kMaxSegments = 1024;
// Steps per lane in the split's aggregate pass (a multiple of kK).
#ifndef SSM_SCAN_AGG_K
#define SSM_SCAN_AGG_K 16
#endif
constexpr int kAggK = SSM_SCAN_AGG_K;
static_assert(kAggK % kK == 0, "aggregate chunks are whole main-pass chunks");
// Steps per lane in the checkpoint-only pass (no readout either, so the
// longer fold fits); a 64-step checkpoint falls on every (64 / K)-th lane.
// The exact zero-order-hold form keeps K = 8 in both passes: at 16 its
// fp32 instantiations would spill.
#ifndef SSM_SCAN_CKPT_K
#define SSM_SCAN_CKPT_K 16
#endif
constexpr int kCkptK = SSM_SCAN_CKPT_K;
static_assert(kAggK % kCkptK == 0, "checkpoint-pass segments are whole chunks");
// Occupancy target (waves per SIMD): 4, which is also what the ~36 KB of LDS
// per 4-wave workgroup allows (4 workgroups per CU).  More resident waves
// were measured not to help: the state loop runs near the VALU issue limit.
template <typename Tin>
constexpr int kMinWavesPerSimd = sizeof(Tin) == 2 ? SSM_SCAN_MINW_BF16 : SSM_SCAN_MINW_F32;

struct ScanParams {
    int dim, seqlen;
    // Layout in elements: every row of x, dt, z, y (one channel) and of Bm,
    // Cm (one state) holds seqlen contiguous steps; rows of a batch entry are
    // `row` apart (x, dt, z, y share it), batch entries are `*_b` apart.
    long long row, x_b, dt_b, z_b, y_b, bc_row, B_b, C_b;
    const void *x, *dt;
    const float *dt_bias, *A;
    const void *Bm, *Cm;
    const float *Dskip;
    const void *z;
    const float *h0;
    void *y;
    float *hL;
    float *ck;  // optional: state entering every 64-step chunk, [batch][dim][nck][N]
    int nck;
    // Sequence split: segment blockIdx.z covers steps [z seg_len, (z+1) seg_len).
    // agg[s][b][d][0..N-1]: state at the end of segment s (from h0 for s = 0,
    // from zero otherwise); agg[s][b][d][N]: sum of Delta over segment s.
    int seg_len, nseg;
    float *agg;
};

__device__ inline bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

template <typename Tin, typename Tout, int N, int K, bool kZoh, bool kCkpt, bool kAgg, bool kOut>
__global__ __launch_bounds__(kThreads, kMinWavesPerSimd<Tin>) void scan_fwd_kernel(ScanParams p)
{
    static_assert(K % 8 == 0, "K must be a multiple of 8");
    static_assert(!(kCkpt && kAgg), "the aggregate pass writes no checkpoints");
    static_assert(kOut || (kCkpt && !kAgg), "a main pass without output writes checkpoints");
    // kRead: the readout (Cm, z, the replay, y); off in the aggregate pass and
    // in the checkpoint-only pass the backward uses
    constexpr bool kRead = !kAgg && kOut;
    static_assert(N * kRow <= kThreads, "one staging slot per thread");
    constexpr int T = kRow * K;  // timesteps per chunk
    constexpr int Q = K / 4;     // float4 per lane per state
    constexpr int NP = N + 1;    // per-channel stride of sA / sCarry (one pad entry)

    // Bm/Cm chunk in LDS, fp32, layout [n][q][lane j] of float4 so that the
    // 16 lanes of a row read 256 contiguous bytes per ds_read_b128.
    // sB has one spare state so the look-ahead load of the last state stays
    // inside the array.
    __shared__ float4 sB[2][(N + 1) * Q * kRow];
    __shared__ float4 sC[2][kRead ? N * Q * kRow : 1];
    // Per channel: NP entries of A * log2(e), then NP entries of the state
    // entering the current chunk.
    __shared__ float sAC[kChannels * 2 * NP];
    // Checkpoints: every 64 steps, kPer per chunk.  The first is the carry
    // entering the chunk; the others are the end states of every kG-th lane,
    // gathered per channel (kMid rows of NP) so that a row of N states goes
    // out in one store instruction.
    static_assert(!kCkpt || (kCkptSteps % K == 0 && T % kCkptSteps == 0), "whole lanes per checkpoint");
    constexpr int kG = kCkptSteps / K;         // lanes per 64-step checkpoint
    constexpr int kPer = T / kCkptSteps;       // checkpoints per chunk
    constexpr int kMid = kPer - 1;             // ... after the chunk's entry
    __shared__ float sMid[kCkpt ? kChannels * kMid * NP : 1];

    const int tid = threadIdx.x;
    const int j = tid & (kRow - 1);
    const int c = tid / kRow;                 // channel within the workgroup
    const int b = blockIdx.y;
    const int dim = p.dim;
    const int seg = blockIdx.z;
    const int lseg = seg * p.seg_len;              // first step of this segment
    const int L = min(p.seqlen - lseg, p.seg_len);  // steps in this segment
    const int d = blockIdx.x * kChannels + c;
    const bool live = d < dim;
    const int dc = live ? d : dim - 1;

    // Wave-uniform row base (its first channel, clamped) and per-lane offset.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d0 = min(int(blockIdx.x) * kChannels + wave * 4, dim - 1);
    const size_t row0 = size_t(d0) * size_t(p.row) + size_t(lseg);
    const Tin *xw = static_cast<const Tin *>(p.x) + size_t(b) * size_t(p.x_b) + row0;
    const Tin *dtw = static_cast<const Tin *>(p.dt) + size_t(b) * size_t(p.dt_b) + row0;
    const Tin *zw = p.z ? static_cast<const Tin *>(p.z) + size_t(b) * size_t(p.z_b) + row0 : nullptr;
    Tout *yw = static_cast<Tout *>(p.y) + size_t(b) * size_t(p.y_b) + row0;
    const uint32_t lane_row = uint32_t(dc - d0) * uint32_t(p.row);  // elements
    // Checkpoint rows: a wave-uniform base at the wave's first channel and a
    // 32-bit lane offset (under 4 nck N <= 2^28 floats).
    [[maybe_unused]] float *ckw = kCkpt ? p.ck + (size_t(b) * dim + d0) * size_t(p.nck) * N : nullptr;
    [[maybe_unused]] const uint32_t ck_lane = uint32_t(dc - d0) * uint32_t(p.nck) * uint32_t(N) + uint32_t(j);
    const Tin *Bb = static_cast<const Tin *>(p.Bm) + size_t(b) * size_t(p.B_b) + size_t(lseg);
    const Tin *Cb = static_cast<const Tin *>(p.Cm) + size_t(b) * size_t(p.C_b) + size_t(lseg);
    // Wave-uniform: every row of every streamed tensor starts on a 16-byte
    // boundary, so all runs of a chunk that lies inside the sequence can use
    // unguarded 16-byte vector accesses.
    const bool rows_vec = aligned16(xw) && aligned16(dtw) && aligned16(Bb) &&
                          (size_t(p.row) * sizeof(Tin)) % 16 == 0 &&
                          (size_t(p.bc_row) * sizeof(Tin)) % 16 == 0 &&
                          (!kRead || ((!zw || aligned16(zw)) && aligned16(yw) && aligned16(Cb) &&
                                      (size_t(p.row) * sizeof(Tout)) % 16 == 0));
    auto chunk_full = [&](int chunk) { return rows_vec && (chunk + 1) * T <= L; };

    for (int s = tid; s < kChannels * NP; s += kThreads) {
        const int cc = s / NP, n = s % NP;
        const int dd = min(int(blockIdx.x) * kChannels + cc, dim - 1);
        sAC[cc * 2 * NP + n] = (n < N) ? p.A[size_t(dd) * N + n] * kLog2e : 0.0f;
    }
    {
        // State entering the segment: h0 for the first; otherwise the
        // segments before it composed in order, h <- exp(A sum Delta) h + end
        // state (each segment's map is affine in its entering state), lane j
        // of the channel's row composing state j.
        // With a split, the aggregate pass copies h0 into the last plane of
        // agg and the main pass reads that copy, so that hL may overwrite h0
        // while other segments of the same channel are still running.
        float *hin = sAC + c * 2 * NP + NP;
        float *h0copy = p.nseg > 1 ? p.agg + ((size_t(p.nseg - 1) * gridDim.y + b) * dim + dc) * NP
                                   : nullptr;
        if (seg == 0 || kAgg) {
            if (j == 0) {
                const bool copy = !kAgg && h0copy;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float v = (p.h0 && seg == 0)
                                        ? (copy ? h0copy[n] : p.h0[(size_t(b) * dim + dc) * N + n])
                                        : 0.0f;
                    hin[n] = v;
                    if (kAgg && seg == 0 && p.h0 && live) h0copy[n] = v;
                }
            }
        } else if (j < N) {
            const float a = p.A[size_t(dc) * N + j] * kLog2e;
            float h = 0.0f;
            for (int s = 0; s < seg; ++s) {
                const float *ag = p.agg + ((size_t(s) * gridDim.y + b) * dim + dc) * NP;
                h = __builtin_fmaf(exp2_hw(a * ag[N]), h, ag[j]);
            }
            hin[j] = h;
        }
        if (j == 0) hin[N] = 0.0f;
    }

    // Staging slot of this thread: state sn, lane block sj (threads < N*16).
    const bool stager = tid < N * kRow;
    const int sn = stager ? tid / kRow : 0, sj = tid % kRow;
    raw_run<Tin, K> stB, stC;
    auto stage_load = [&](const Tin *src, int chunk, raw_run<Tin, K> &st) {
        const int l = chunk * T + sj * K;
        const Tin *q = src + size_t(sn) * size_t(p.bc_row) + l;
        if (chunk_full(chunk)) {
            load_raw<Tin, K, true>(q, true, K, st);
        } else {
            const int cnt = max(0, min(K, L - l));
            load_raw<Tin, K, true>(q, cnt == K && aligned16(q), cnt, st);
        }
    };
    auto stage_store = [&](float4 *dst, const raw_run<Tin, K> &st) {
        float v[K];
        decode_raw<Tin, K>(st, v);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            dst[(sn * Q + q) * kRow + sj] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    };

    raw_run<Tin, K> rx, rdt, rz;
    auto xd_load = [&](int chunk) {
        const int l = chunk * T + j * K;
        const uint32_t off = (lane_row + uint32_t(l)) * uint32_t(sizeof(Tin));
        const Tin *qx = at(xw, off), *qd = at(dtw, off);
        if (chunk_full(chunk)) {
            load_raw<Tin, K>(qx, true, K, rx);
            load_raw<Tin, K>(qd, true, K, rdt);
        } else {
            const int cnt = max(0, min(K, L - l));
            const bool vec = cnt == K && aligned16(qx) && aligned16(qd);
            load_raw<Tin, K>(qx, vec, cnt, rx);
            load_raw<Tin, K>(qd, vec, cnt, rdt);
        }
    };
    auto z_load = [&](int chunk, uint32_t off) {
        const Tin *qz = at(zw, off);
        if (chunk_full(chunk)) {
            load_raw<Tin, K>(qz, true, K, rz);
        } else {
            const int cnt = max(0, min(K, L - (chunk * T + j * K)));
            load_raw<Tin, K>(qz, cnt == K && aligned16(qz), cnt, rz);
        }
    };

    const int nchunks = (L + T - 1) / T;
    if (stager) {
        stage_load(Bb, 0, stB);
        if constexpr (kRead) stage_load(Cb, 0, stC);
        stage_store(sB[0], stB);
        if constexpr (kRead) stage_store(sC[0], stC);
    }
    xd_load(0);
    lds_barrier();

    float *aptr = sAC + c * 2 * NP;  // A' at aptr[n], carry at aptr[NP + n]
    [[maybe_unused]] float dtot = 0.0f;  // this lane's Delta sum (aggregate pass)

    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        const int l0 = ch * T + j * K;
        const int cnt = max(0, min(K, L - l0));
        const uint32_t yoff = (lane_row + uint32_t(l0)) * uint32_t(sizeof(Tin));

        // Delta, Delta*x and the skip term for this lane's K steps; steps past
        // the end of the sequence get Delta = 0 (identity map: a = 1, b = 0).
        const bool full = chunk_full(ch);
        float delta[K], u[K], yv[K];
        [[maybe_unused]] float invd[K];  // 1/Delta (exact-ZOH B-bar only)
        float sumd = 0.0f;
        const float bias = p.dt_bias ? p.dt_bias[dc] : 0.0f;
        const float skip = p.Dskip ? p.Dskip[dc] : 0.0f;
        if (full) {
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const float xv = decode_raw_at<Tin, K>(rx, i);
                delta[i] = softplus(decode_raw_at<Tin, K>(rdt, i) + bias);
                u[i] = delta[i] * xv;
                yv[i] = skip * xv;
                sumd += delta[i];
                if constexpr (kZoh) invd[i] = rcp_hw(delta[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const float xv = decode_raw_at<Tin, K>(rx, i);
                const float dv = softplus(decode_raw_at<Tin, K>(rdt, i) + bias);
                const bool in = i < cnt;
                delta[i] = in ? dv : 0.0f;
                u[i] = in ? dv * xv : 0.0f;
                yv[i] = skip * xv;
                sumd += delta[i];
                if constexpr (kZoh) invd[i] = in ? rcp_hw(dv) : 0.0f;
            }
        }
        const bool more = ch + 1 < nchunks;
        // Checkpoints for the backward pass: the state entering each 64-step
        // part of the chunk, one (b, d, part) row of N states per store
        // instruction (lane j writes state j), so every row goes out as one
        // contiguous line instead of N scattered words.
        [[maybe_unused]] auto store_ck = [&](const float *src, int part) {
            static_assert(N <= kRow, "one lane per state");
            const int ck = kPer * (ch + lseg / T) + part;  // global 64-step chunk
            if (live && j < N && ck < p.nck) ckw[ck_lane + uint32_t(ck) * uint32_t(N)] = src[j];
        };
        if constexpr (kCkpt) store_ck(aptr + NP, 0);  // the carry entering the chunk

        const float4 *bp = sB[buf] + j;
        const float4 *cp = sC[buf] + j;
        float bv[K];
        auto load_b = [&](const float4 *src, float *v) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float4 w = src[q * kRow];
                v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
            }
        };
        load_b(bp, bv);
        float ap = aptr[0];
        float carry = aptr[NP];

        // One state: local fold, row scan, carry update and replay.
        auto state_step = [&](int n) {
            float cv[K];
            if constexpr (kRead) {
                load_b(cp, cv);
                cp += Q * kRow;
            }
            float dA[K], bb[K];
            if constexpr (kZoh) {
                // exact zero-order hold: B-bar x = phi(Delta A) Delta B x
                const float inva = rcp_hw(ap) * kLog2e;  // 1/A
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    const float t = delta[i] * ap;
                    dA[i] = exp2_hw(t);
                    bb[i] = (u[i] * bv[i]) * phi_zoh(t * kLn2, dA[i], invd[i] * inva);
                }
            } else {
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    dA[i] = exp2_hw(delta[i] * ap);
                    bb[i] = u[i] * bv[i];
                }
            }
            float hl = bb[0];
#pragma unroll
            for (int i = 1; i < K; ++i) hl = __builtin_fmaf(dA[i], hl, bb[i]);
            float aa = exp2_hw(sumd * ap);
            float hend, h = carry;
            row_scan(aa, hl, hend, h);
            if (j == kRow - 1) aptr[NP + n] = hend;
            if constexpr (kCkpt) {
                // entering the next 64-step part of the chunk
                if ((j + 1) % kG == 0 && j < kRow - 1) sMid[(c * kMid + (j + 1) / kG - 1) * NP + n] = hend;
            }
            bp += Q * kRow;
            load_b(bp, bv);          // next state's B (one past the end on the last state)
            ap = aptr[n + 1];
            carry = aptr[NP + n + 1];
            if constexpr (kRead) {
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    h = __builtin_fmaf(dA[i], h, bb[i]);
                    yv[i] = __builtin_fmaf(cv[i], h, yv[i]);
                }
            }
        };

        // Two states at once (the two-states-per-trip instantiation): both
        // folds first, then one asm block in which the two DPP scans cover
        // each other's read hazards (no wait states), then both replays.
        [[maybe_unused]] auto state_pair = [&](int n) {
            float bv1[K];
            load_b(bp + Q * kRow, bv1);
            const float ap1 = aptr[n + 1], carry1 = aptr[NP + n + 1];
            float dA0[K], bb0[K], dA1[K], bb1[K];
#pragma unroll
            for (int i = 0; i < K; ++i) {
                dA0[i] = exp2_hw(delta[i] * ap);
                bb0[i] = u[i] * bv[i];
            }
#pragma unroll
            for (int i = 0; i < K; ++i) {
                dA1[i] = exp2_hw(delta[i] * ap1);
                bb1[i] = u[i] * bv1[i];
            }
            float hl0 = bb0[0], hl1 = bb1[0];
#pragma unroll
            for (int i = 1; i < K; ++i) {
                hl0 = __builtin_fmaf(dA0[i], hl0, bb0[i]);
                hl1 = __builtin_fmaf(dA1[i], hl1, bb1[i]);
            }
            float aa0 = exp2_hw(sumd * ap), aa1 = exp2_hw(sumd * ap1);
            float hend0, hend1, h0 = carry, h1 = carry1;
            row_scan_x2(aa0, hl0, hend0, h0, aa1, hl1, hend1, h1);
            if (j == kRow - 1) {
                aptr[NP + n] = hend0;
                aptr[NP + n + 1] = hend1;
            }
            bp += 2 * Q * kRow;
            load_b(bp, bv);  // the next pair's first B (one past the end after the last)
            ap = aptr[n + 2];
            carry = aptr[NP + n + 2];
            if constexpr (kRead) {
                // each state's Cm run is read just before its replay, so that
                // neither is held across the folds and the scan
                float cv[K];
                load_b(cp, cv);
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    h0 = __builtin_fmaf(dA0[i], h0, bb0[i]);
                    yv[i] = __builtin_fmaf(cv[i], h0, yv[i]);
                }
                load_b(cp + Q * kRow, cv);
                cp += 2 * Q * kRow;
#pragma unroll
                for (int i = 0; i < K; ++i) {
                    h1 = __builtin_fmaf(dA1[i], h1, bb1[i]);
                    yv[i] = __builtin_fmaf(cv[i], h1, yv[i]);
                }
            }
        };

        // The loads in flight are spread over thirds of the states so that
        // few of them hold registers at once: the next chunk's Bm and Cm are
        // staged during the first third; this chunk's z and the next chunk's
        // x and dt are fetched during the last third.
        if constexpr (N >= 8) {
            constexpr int N1 = (N + 2) / 3, N2 = N - (N + 2) / 3;
            // Two states per loop trip (state_pair: shared LDS address
            // updates, the two DPP scans interleaved with no wait states):
            // measured in interleaved runs against one state per trip
            // (SSM_SCAN_PAIRS=0), 1.5 % faster at the 130M-layer shape and
            // equal within noise at the 2.8B layer.  The other variants
            // would spill at that unroll, so they keep one.
            constexpr int kSU =
                (SSM_SCAN_PAIRS && K == 8 && sizeof(Tin) == 2 && N == 16 && !kZoh && !kCkpt && kRead) ? 2 : 1;
            if (more && stager) {
                stage_load(Bb, ch + 1, stB);
                if constexpr (kRead) stage_load(Cb, ch + 1, stC);
            }
            if constexpr (kSU == 2) {
                static_assert(N1 % 2 == 0 && N2 % 2 == 0 && N % 2 == 0, "whole pairs per third");
#pragma unroll 1
                for (int n = 0; n < N1; n += 2) state_pair(n);
                if (more && stager) {
                    stage_store(sB[buf ^ 1], stB);
                    if constexpr (kRead) stage_store(sC[buf ^ 1], stC);
                }
#pragma unroll 1
                for (int n = N1; n < N2; n += 2) state_pair(n);
                if (kRead && zw) z_load(ch, yoff);
                if (more) xd_load(ch + 1);
#pragma unroll 1
                for (int n = N2; n < N; n += 2) state_pair(n);
            } else {
#pragma unroll 1
                for (int n = 0; n < N1; ++n) state_step(n);
                if (more && stager) {
                    stage_store(sB[buf ^ 1], stB);
                    if constexpr (kRead) stage_store(sC[buf ^ 1], stC);
                }
#pragma unroll 1
                for (int n = N1; n < N2; ++n) state_step(n);
                if (kRead && zw) z_load(ch, yoff);
                if (more) xd_load(ch + 1);
#pragma unroll 1
                for (int n = N2; n < N; ++n) state_step(n);
            }
        } else {
            // few states: everything is fetched up front
            if (more && stager) {
                stage_load(Bb, ch + 1, stB);
                if constexpr (kRead) stage_load(Cb, ch + 1, stC);
            }
            if (kRead && zw) z_load(ch, yoff);
            if (more) xd_load(ch + 1);
#pragma unroll 1
            for (int n = 0; n < N; ++n) state_step(n);
            if (more && stager) {
                stage_store(sB[buf ^ 1], stB);
                if constexpr (kRead) stage_store(sC[buf ^ 1], stC);
            }
        }

        if constexpr (kAgg) dtot += sumd;
        if (kRead && zw) {
#pragma unroll
            for (int i = 0; i < K; ++i) yv[i] *= silu(decode_raw_at<Tin, K>(rz, i));
        }
        if (kRead && live) {
            Tout *yr = at(yw, uint32_t((lane_row + uint32_t(l0)) * sizeof(Tout)));
            if (full)
                store_y<Tout, K>(yr, true, K, yv);
            else if (cnt > 0)
                store_y<Tout, K>(yr, cnt == K && aligned16(yr), cnt, yv);
        }
        if constexpr (kCkpt) {
            // written by lanes of the same row (same wave) in the state loop
#pragma unroll
            for (int m = 0; m < kMid; ++m) store_ck(sMid + (c * kMid + m) * NP, m + 1);
        }
        lds_barrier();
    }

    if constexpr (kAgg) {
        // the segment's Delta sum over the row's 16 lanes
#pragma unroll
        for (int m = 1; m < kRow; m <<= 1) dtot += __shfl_xor(dtot, m, kRow);
        if (live && j == 0) {
            float *ag = p.agg + ((size_t(seg) * gridDim.y + b) * dim + d) * NP;
#pragma unroll
            for (int n = 0; n < N; ++n) ag[n] = aptr[NP + n];
            ag[N] = dtot;
        }
    } else if (p.hL && live && j == 0 && seg == int(gridDim.z) - 1) {
#pragma unroll
        for (int n = 0; n < N; ++n) p.hL[(size_t(b) * dim + d) * N + n] = aptr[NP + n];
    }
}

template <typename Tin, typename Tout, int N, bool kZoh>
hipError_t launch_typed(const ScanArgs &a, hipStream_t stream)
{
    constexpr int K = kK;
    const ScanSplit sp = scan_fwd_split(a.batch, a.dim, a.seqlen);
    ScanParams p{a.dim, a.seqlen, a.row, a.x_b, a.dt_b, a.z_b, a.y_b, a.bc_row, a.B_b, a.C_b,
                 a.x, a.dt, a.dt_bias, a.A, a.Bm, a.Cm,
                 a.Dskip, a.z, a.h0, a.y, a.hL, a.ck, (a.seqlen + kCkptSteps - 1) / kCkptSteps,
                 sp.seg_len, sp.nseg, a.agg};
    const unsigned gx = (unsigned(a.dim) + kChannels - 1) / kChannels;
    if (log_enabled() && sp.nseg > 1)
        log_line("scan_fwd: sequence split into %d segments of %d steps; aggregate pass "
                 "scan_fwd_kernel<in %s, N %d, K %d, zoh %d, aggregate>, grid (%u, %d, %d) x %d threads",
                 sp.nseg, sp.seg_len, type_tag<Tin>(), N, kZoh ? kK : kAggK, int(kZoh), gx, a.batch,
                 sp.nseg - 1, kThreads);
    if (sp.nseg > 1) {
        // every segment but the last: its end state and Delta sum
        // The aggregate pass has no replay, so each lane's fold streams its
        // steps and 16 steps per lane fit: half the row scans per element.
        hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, N, kZoh ? kK : kAggK, kZoh, false, true, true>),
                           dim3(gx, a.batch, sp.nseg - 1), dim3(kThreads), 0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid(gx, a.batch, sp.nseg);
    if (log_enabled())
        log_line("scan_fwd: scan_fwd_kernel<in %s, out %s, N %d, K %d, zoh %d, checkpoints %d, "
                 "output %d>, %s, grid (%u, %u, %u) x %d threads",
                 type_tag<Tin>(), type_tag<Tout>(), N, (a.ckpt_only && !kZoh) ? kCkptK : K, int(kZoh),
                 a.ck ? 1 : 0, a.ckpt_only ? 0 : 1, sp.nseg > 1 ? "main pass" : "no split", grid.x, grid.y,
                 grid.z, kThreads);
    if (a.ckpt_only) {
        // no output: one instantiation (fp32 Tout) serves every caller
        if constexpr (sizeof(Tout) == 4) {
            hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, N, kZoh ? kK : kCkptK, kZoh, true, false, false>),
                               grid, dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (a.ck) {
        hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, N, K, kZoh, true, false, true>), grid,
                           dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, N, K, kZoh, false, false, true>), grid, dim3(kThreads),
                       0, stream, p);
    return hipGetLastError();
}

template <typename Tin, typename Tout, bool kZoh>
hipError_t launch_n(const ScanArgs &a, hipStream_t stream)
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
hipError_t launch_mode(const ScanArgs &a, hipStream_t stream)
{
    return a.zoh ? launch_n<Tin, Tout, true>(a, stream) : launch_n<Tin, Tout, false>(a, stream);
}

}  // namespace

ScanSplit scan_fwd_split(int batch, int dim, int seqlen)
{
    constexpr int T = kRow * kAggK;  // segments: whole chunks of both passes
    const long long wgs = (long long)batch * (((long long)dim + kChannels - 1) / kChannels);
    ScanSplit sp{1, seqlen};
    if (wgs >= SSM_SPLIT_BELOW_WGS) return sp;
    long long nseg = kSplitTargetWgs / wgs;  // whole multiples of the workgroups
    nseg = std::min<long long>(nseg, seqlen / SSM_SPLIT_MIN_STEPS);
    nseg = std::min<long long>(nseg, kMaxSegments);
    if (nseg < 2) return sp;
    const long long per = (seqlen + nseg - 1) / nseg;
    sp.seg_len = int((per + T - 1) / T * T);
    sp.nseg = int((seqlen + sp.seg_len - 1) / sp.seg_len);
    if (sp.nseg < 2) sp = {1, seqlen};
    return sp;
}

size_t scan_fwd_split_bytes(int batch, int dim, int seqlen, int dstate)
{
    const ScanSplit sp = scan_fwd_split(batch, dim, seqlen);
    if (sp.nseg < 2) return 0;
    return size_t(sp.nseg) * size_t(batch) * size_t(dim) * size_t(dstate + 1) * sizeof(float);
}

hipError_t launch_scan_fwd(const ScanArgs &a, hipStream_t stream)
{
    if (a.in_bf16) {
        return a.out_bf16 ? launch_mode<bf16_t, bf16_t>(a, stream)
                          : launch_mode<bf16_t, float>(a, stream);
    }
    return a.out_bf16 ? launch_mode<float, bf16_t>(a, stream) : launch_mode<float, float>(a, stream);
}

}  // namespace ssm
