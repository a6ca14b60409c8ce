// ssm_device.hpp -- device helpers shared by the scan and decode kernels.
//
// Input widening, the two pointwise functions of the selective scan
// (softplus for the step size, silu for the output gate) built on the
// hardware base-2 exponential and logarithm, and the DPP lane moves used by
// the in-row associative scan.  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- storage types
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {
    uint16_t bits;
};

template <typename T> struct io;

template <> struct io<float> {
    // elements per 16-byte vector
    static constexpr int kVec = 4;
    __device__ static inline float load1(const float *p) { return *p; }
    // decode one 16-byte vector into 4 floats
    __device__ static inline void unpack(const u32x4 &v, float *out)
    {
        out[0] = __uint_as_float(v.x);
        out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z);
        out[3] = __uint_as_float(v.w);
    }
};

template <> struct io<bf16_t> {
    static constexpr int kVec = 8;
    // bf16 -> fp32 is exact: the 16 bits become the high half of the fp32 word
    __device__ static inline float load1(const bf16_t *p)
    {
        return __uint_as_float(uint32_t(p->bits) << 16);
    }
    __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    __device__ static inline void unpack(const u32x4 &v, float *out)
    {
        out[0] = lo(v.x); out[1] = hi(v.x);
        out[2] = lo(v.y); out[3] = hi(v.y);
        out[4] = lo(v.z); out[5] = hi(v.z);
        out[6] = lo(v.w); out[7] = hi(v.w);
    }
};

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Load `n` consecutive elements starting at p (n a multiple of the vector
// width) as fp32.  `vec` selects 16-byte vector loads; otherwise element
// loads guarded by `count` (elements at index >= count read as 0).
template <typename T, int n>
__device__ inline void load_run(const T *p, bool vec, int count, float *out)
{
    static_assert(n % io<T>::kVec == 0, "a run must be whole 16-byte vectors");
    if (vec) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int v = 0; v < n / io<T>::kVec; ++v) {
            u32x4 w = __builtin_nontemporal_load(q + v);
            io<T>::unpack(w, out + v * io<T>::kVec);
        }
    } else {
#pragma unroll
        for (int i = 0; i < n; ++i) out[i] = (i < count) ? io<T>::load1(p + i) : 0.0f;
    }
}

// Raw (undecoded) form of the same load, so that a prefetch can keep the
// data in its compact storage form until it is used.
template <typename T, int n> struct raw_run {
    static constexpr int kWords = n * int(sizeof(T)) / 4;
    uint32_t w[kWords];
};

// Streamed data (read once) takes nontemporal loads; kShared = true takes
// ordinary cached loads, for data that other workgroups read at about the
// same time (Bm and Cm, shared by every channel of a batch row).
template <typename T, int n, bool kShared = false>
__device__ inline void load_raw(const T *p, bool vec, int count, raw_run<T, n> &r)
{
    static_assert(n % io<T>::kVec == 0, "a run must be whole 16-byte vectors");
    if (vec) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int v = 0; v < raw_run<T, n>::kWords / 4; ++v) {
            u32x4 x = kShared ? q[v] : __builtin_nontemporal_load(q + v);
            r.w[4 * v + 0] = x.x; r.w[4 * v + 1] = x.y;
            r.w[4 * v + 2] = x.z; r.w[4 * v + 3] = x.w;
        }
    } else {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < n; ++i)
                r.w[i] = (i < count) ? reinterpret_cast<const uint32_t *>(p)[i] : 0u;
        } else {
            const uint16_t *s = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
            for (int i = 0; i < n; i += 2) {
                uint32_t lo = (i < count) ? s[i] : 0u;
                uint32_t hi = (i + 1 < count) ? s[i + 1] : 0u;
                r.w[i / 2] = lo | (hi << 16);
            }
        }
    }
}

template <typename T, int n>
__device__ inline void decode_raw(const raw_run<T, n> &r, float *out)
{
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < n; ++i) out[i] = __uint_as_float(r.w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            out[2 * i] = io<bf16_t>::lo(r.w[i]);
            out[2 * i + 1] = io<bf16_t>::hi(r.w[i]);
        }
    }
}

template <typename T, int n>
__device__ inline float decode_raw_at(const raw_run<T, n> &r, int i)
{
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(r.w[i]);
    } else {
        return (i & 1) ? io<bf16_t>::hi(r.w[i / 2]) : io<bf16_t>::lo(r.w[i / 2]);
    }
}

// ---------------------------------------------------------------- pointwise math
__device__ inline float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ inline float log2_hw(float v) { return __builtin_amdgcn_logf(v); }
__device__ inline float rcp_hw(float v) { return __builtin_amdgcn_rcpf(v); }

// softplus(u) = ln(1 + e^u) = max(u, 0) + log1p(e^-|u|).
// With t = e^-|u| in (0, 1] and w = fl(1 + t), the rounding error of w is
// c = t - (w - 1) exactly (w - 1 is exact for w in [1, 2]); then
// log1p(t) = ln(w) + ln(1 + c/w) ~= ln(w) + c, whose dropped term is below
// 2^-24 t relative.  This keeps full relative accuracy for tiny t, where a
// plain log(1 + t) would lose it.
__device__ inline float softplus(float u)
{
    const float t = exp2_hw(-fabsf(u) * kLog2e);
    const float w = 1.0f + t;
    const float c = t - (w - 1.0f);
    const float l = __builtin_fmaf(log2_hw(w), kLn2, c);
    return fmaxf(u, 0.0f) + l;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).  For z -> -inf the exponential
// overflows to +inf and the reciprocal to 0, giving -0.
__device__ inline float silu(float z)
{
    return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// phi(x) = (e^x - 1) / x, the factor that turns Delta*B into the exact
// zero-order-hold B-bar = (Delta A)^-1 (exp(Delta A) - 1) Delta B = phi(Delta A) Delta B.
// `abar` = e^x (already computed for A-bar) and inv_x = 1/x.  For |x| < 1/16
// the Taylor series to x^4 (truncation below 1e-9 relative) avoids the
// cancellation in abar - 1; elsewhere (abar - 1) / x is accurate to ~1e-6.
// The select keeps x = 0 (A = 0 or Delta = 0) finite: phi(0) = 1.
__device__ inline float phi_zoh(float x, float abar, float inv_x)
{
    float p = __builtin_fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f);
    p = __builtin_fmaf(x, p, 1.0f / 6.0f);
    p = __builtin_fmaf(x, p, 0.5f);
    p = __builtin_fmaf(x, p, 1.0f);
    const float big = (abar - 1.0f) * inv_x;
    return fabsf(x) < 0.0625f ? p : big;
}

// psi(x) = (x e^x - (e^x - 1)) / x^2, the A-derivative factor of the exact
// ZOH input term: d/dA [(e^(Delta A) - 1) / A] = Delta^2 psi(Delta A).  For
// |x| < 1/4 the Taylor series sum_m (m + 1) x^m / (m + 2)! to x^5 (truncation
// below 1e-7 relative) avoids the cancellation of the closed form; elsewhere
// the closed form is accurate to ~1e-5.  psi(0) = 1/2.
__device__ inline float psi_zoh(float x, float abar, float inv_x)
{
    float p = __builtin_fmaf(x, 1.0f / 840.0f, 1.0f / 144.0f);
    p = __builtin_fmaf(x, p, 1.0f / 30.0f);
    p = __builtin_fmaf(x, p, 0.125f);
    p = __builtin_fmaf(x, p, 1.0f / 3.0f);
    p = __builtin_fmaf(x, p, 0.5f);
    const float big = __builtin_fmaf(x, abar, 1.0f - abar) * inv_x * inv_x;
    return fabsf(x) < 0.25f ? p : big;
}

// ---------------------------------------------------------------- DPP lane moves
// dpp_ctrl encodings (GFX9 DPP): row_shr:s = 0x110 + s within a 16-lane row;
// row_newbcast:k = 0x150 + k broadcasts lane k of each row to the whole row.
template <int kCtrl>
__device__ inline float dpp(float old_value, float src)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old_value),
                                           __builtin_bit_cast(int, src), kCtrl, 0xF, 0xF, false));
}

template <int kShift> __device__ inline float row_shr(float identity, float v)
{
    static_assert(kShift >= 1 && kShift <= 15, "row_shr range");
    return dpp<0x110 + kShift>(identity, v);
}

__device__ inline float row_bcast_last(float v) { return dpp<0x15F>(v, v); }

}  // namespace ssm
