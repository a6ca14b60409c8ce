// scan_common.hpp -- pieces shared by the scan kernels (forward, chunk
// states, backward): an LDS-only workgroup barrier, the in-row DPP scans of
// affine maps in forward and reverse time, and run stores.  gfx950 only.
#pragma once

#include "ssm_device.hpp"

namespace ssm {

// Workgroup barrier that orders LDS only.  __syncthreads() would also wait
// for every outstanding global load and store of the wave (s_waitcnt vmcnt),
// which here would cut the prefetch of the next chunk short at each chunk
// boundary.  Waves exchange data only through LDS, so LDS ordering suffices.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive scan of affine maps h -> a h + b over the 16 lanes of each DPP
// row, then the state at the end (hend) and at the start (h) of every lane's
// block given the state entering the chunk (passed in h).  Level s combines
// lane j with lane j - s, whose map covers earlier steps and is applied
// first: (a, b) <- (a_{j-s} a, b_{j-s} a + b).  Lanes with no partner inside
// the row are left unwritten (bound_ctrl off), i.e. combined with the
// identity map.  Lane 0 of each row keeps the carry as its start state.
// Each v_*_dpp reads its DPP source at least two wait states after that
// register was last written (the GFX9 VALU-write -> DPP-read hazard), hence
// the s_nop padding.  All 64 lanes must be active.
__device__ inline void row_scan(float &a, float &b, float &hend, float &h)
{
    // on entry h holds the carry; v_fma reads it before v_mov_dpp overwrites it
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
        "v_fma_f32 %2, %0, %3, %1\n\t"
        "s_nop 1\n\t"
        "v_mov_b32_dpp %3, %2 row_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(a), "+v"(b), "=&v"(hend), "+v"(h));
}

// Two independent row scans (see row_scan), interleaved so that each one's
// DPP read hazard is covered by the other's instructions instead of wait
// states.
__device__ inline void row_scan_x2(float &a0, float &b0, float &e0, float &h0,
                                   float &a1, float &b1, float &e1, float &h1)
{
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %4, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %4 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %4, %4 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %4 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %4, %4 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %4 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %4, %4 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fma_f32 %2, %0, %3, %1\n\t"
        "v_fma_f32 %6, %4, %7, %5\n\t"
        "s_nop 0\n\t"
        "v_mov_b32_dpp %3, %2 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %7, %6 row_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(a0), "+v"(b0), "=&v"(e0), "+v"(h0), "+v"(a1), "+v"(b1), "=&v"(e1), "+v"(h1));
}

template <typename Tout, int K>
__device__ inline void store_y(Tout *dst, bool vec, int count, const float *v)
{
    static_assert(K % (16 / sizeof(Tout)) == 0, "a run must be whole 16-byte vectors");
    if constexpr (sizeof(Tout) == 4) {
        if (vec) {
            f32x4 *q = reinterpret_cast<f32x4 *>(dst);
#pragma unroll
            for (int i = 0; i < K / 4; ++i) {
                f32x4 w = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
                q[i] = w;
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
                q[i] = w;
            }
        } else {
            uint16_t *s = reinterpret_cast<uint16_t *>(dst);
#pragma unroll
            for (int i = 0; i < K; ++i)
                if (i < count) s[i] = uint16_t(pack_bf16x2(v[i], 0.0f) & 0xffffu);
        }
    }
}

// Global access through a wave-uniform base and a 32-bit per-lane byte
// offset, so that only one VGPR per access stream is spent on addressing.
template <typename T>
__device__ inline const T *at(const T *base, uint32_t byte_off)
{
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}
template <typename T>
__device__ inline T *at(T *base, uint32_t byte_off)
{
    return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + byte_off);
}

// Mirror image of row_scan for recurrences that run backwards in time
// (mu_out = P mu_in + Q per lane, mu entering from the right): level s
// combines lane j with lane j + s, whose map acts first,
// (P, Q) <- (P P_{j+s}, P Q_{j+s} + Q).  On exit hend = P_incl * carry +
// Q_incl (lane 0: the whole row applied to the carry entering at lane 15)
// and h = the value entering each lane from its right neighbour (lane 15
// keeps the carry).  Same hazard padding; all 64 lanes must be active.
__device__ inline void row_scan_rev(float &a, float &b, float &hend, float &h)
{
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 0\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 0\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 0\n\t"
        "v_fmac_f32_dpp %1, %1, %0 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %0, %0, %0 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fma_f32 %2, %0, %3, %1\n\t"
        "s_nop 1\n\t"
        "v_mov_b32_dpp %3, %2 row_shl:1 row_mask:0xf bank_mask:0xf"
        : "+v"(a), "+v"(b), "=&v"(hend), "+v"(h));
}

}  // namespace ssm
