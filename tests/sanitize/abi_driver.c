/* Drives the host side of the library's C ABI (include/ssm.h, ssm_bwd.h,
 * ssm_conv.h) under AddressSanitizer and UndefinedBehaviorSanitizer (built
 * with the sanitizers on the host pass only and run by
 * tests/test_sanitize.py): the workspace-size queries over ordinary and
 * extreme sizes, and every entry point's argument validation on calls that
 * must be refused.  Device pointers are fake, never-dereferenced addresses;
 * every call here must fail validation (status 1-7), so nothing is launched
 * and no GPU is needed.  An out-of-bounds read of a layout struct, a signed
 * overflow in the size arithmetic or any other undefined behaviour aborts.
 * Written in C, as a C caller of the ABI (where any int is a valid status).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm.h"
#include "ssm_bwd.h"
#include "ssm_conv.h"

static int failures = 0;

#define REFUSED(call)                                                                   \
    do {                                                                                \
        const int st_ = (int)(call);                                                      \
        if (st_ < 1 || st_ > 7) {                                                       \
            fprintf(stderr, "line %d: expected a validation error, got %d\n", __LINE__, st_); \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

static void *fake(int k) { return (void *)(uintptr_t)(0x100000000ull * (unsigned long long)(k + 1)); }

int main(void)
{
    const int big = 65535, maxL = (1 << 28) - 4096;
    const int sizes[][4] = {{1, 1, 1, 1},         {4, 5120, 2048, 16}, {1, 1536, 1 << 20, 16},
                            {1, 16, 2048, 16},    {255, 16, 4096, 4},  {big, 1, 1, 16},
                            {1, 4, maxL, 16},     {1, 1, maxL, 1},     {2, 1 << 30, 64, 16},
                            {big, 1 << 20, 1 << 20, 16}, {0, 1, 1, 1}, {1, -5, 1, 1},
                            {1, 1, maxL + 1, 1},  {1, 1, 1, 3},        {1, 2147483647, 2147483647, 16}};
    size_t sum = 0;
    for (size_t k = 0; k < sizeof sizes / sizeof sizes[0]; ++k) {
        const int *s = sizes[k];
        sum += ssm_scan_fwd_workspace_bytes(s[0], s[1], s[2], s[3]);
        sum += ssm_scan_bwd_workspace_bytes(s[0], s[1], s[2], s[3]);
    }
    for (int st = -1; st < 100; ++st) sum += (size_t)ssm_status_string((ssm_status_t)st)[0];

    void *x = fake(0), *dt = fake(1), *Bm = fake(2), *Cm = fake(3), *z = fake(4), *y = fake(5);
    float *A = (float *)(fake(6)), *h0 = (float *)(fake(7));
    float *hL = (float *)(fake(8)), *bias = (float *)(fake(9));
    float *Dk = (float *)(fake(10)), *ws = (float *)(fake(11));
    const ssm_dtype_t bf = SSM_BF16, f32 = SSM_F32;

    // forward: each case breaks one rule
    REFUSED(ssm_scan_fwd(2, 8, 40, 16, bf, 0, NULL, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(0, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(2, 8, maxL + 1, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(2, 8, 40, 3, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(2, 8, 40, 16, (ssm_dtype_t)9, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(2, 8, 40, 16, bf, 0x80, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(2, 8, 40, 16, bf, 0, (char *)x + 1, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, x, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd(1, 16, 4096, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, NULL, 0, 0));
    REFUSED(ssm_scan_fwd(1, 16, 4096, 16, bf, SSM_FLAG_CHECKPOINTS, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, ws, 16, 0));
    REFUSED(ssm_scan_fwd(big, 1 << 20, 1 << 20, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, 0));
    REFUSED(ssm_scan_fwd_noalloc(2, 8, 40, 16, bf, SSM_FLAG_CHECKPOINTS, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, NULL, 0));
    REFUSED(ssm_scan_fwd_noalloc(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, x, hL, NULL, 0));
    // strided layouts: negative, too small, too large, overflowing spans
    /* per field: negative, below the minimum, past the supported range, and
     * a value whose span overflows 64 bits */
    const long long bad_row[] = {-1, 39, 1ll << 28, 1ll << 62};
    const long long bad_bc_batch[] = {-1, 16 * 40 - 1, 1ll << 56, 1ll << 62};
    const long long bad_seq_batch[] = {-1, 8 * 40 - 1, 1ll << 41, 1ll << 62};
    for (size_t k = 0; k < 4; ++k) {
        ssm_scan_layout_t lay = {0};
        lay.seq_row = bad_row[k];
        REFUSED(ssm_scan_fwd_strided(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, &lay, 0));
        ssm_scan_layout_t lay1 = {0};
        lay1.bc_row = bad_row[k];
        REFUSED(ssm_scan_fwd_strided(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, &lay1, 0));
        ssm_scan_layout_t lay2 = {0};
        lay2.bc_batch[1] = bad_bc_batch[k];
        REFUSED(ssm_scan_fwd_strided(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, &lay2, 0));
        ssm_scan_layout_t lay3 = {0};
        lay3.seq_batch[3] = bad_seq_batch[k];
        REFUSED(ssm_scan_fwd_strided(big, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, y, hL, 0, 0, &lay3, 0));
    }
    // decode step
    float *state = (float *)(fake(12));
    REFUSED(ssm_state_update(64, 5120, 16, bf, 0, NULL, x, dt, bias, A, Bm, Cm, Dk, z, f32, y, 0));
    REFUSED(ssm_state_update(64, 5120, 16, bf, 0, state + 1, x, dt, bias, A, Bm, Cm, Dk, z, f32, y, 0));
    REFUSED(ssm_state_update(big + 1, 5120, 16, bf, 0, state, x, dt, bias, A, Bm, Cm, Dk, z, f32, y, 0));
    REFUSED(ssm_state_update(64, 5120, 16, bf, 4, state, x, dt, bias, A, Bm, Cm, Dk, z, f32, y, 0));
    REFUSED(ssm_state_update(64, 5120, 16, bf, 0, state, x, dt, bias, A, Bm, Cm, Dk, z, f32, state, 0));
    ssm_update_layout_t ul = {0};
    ul.C_batch = -3;
    REFUSED(ssm_state_update_strided(64, 5120, 16, bf, 0, state, x, dt, bias, A, Bm, Cm, Dk, z, f32, y, &ul, 0));
    ul.C_batch = 1ll << 62;
    REFUSED(ssm_state_update_strided(64, 5120, 16, bf, 0, state, x, dt, bias, A, Bm, Cm, Dk, z, f32, y, &ul, 0));
    // conv and its decode step
    float *w = (float *)(fake(13)), *s0 = (float *)(fake(14));
    REFUSED(ssm_conv1d_fwd(4, 5120, 2048, 5, bf, SSM_CONV_SILU, x, w, bias, s0, bf, y, hL, 0));
    REFUSED(ssm_conv1d_fwd(4, 5120, 2048, 4, bf, 0x10, x, w, bias, s0, bf, y, hL, 0));
    REFUSED(ssm_conv1d_fwd(4, 5120, 2048, 4, bf, 0, x, w, bias, s0, bf, x, hL, 0));
    ssm_conv_layout_t cl = {0};
    cl.y_row = 2047;
    REFUSED(ssm_conv1d_fwd_strided(4, 5120, 2048, 4, bf, 0, x, w, bias, s0, bf, y, hL, &cl, 0));
    cl.y_row = 0;
    cl.x_batch = 1ll << 62;
    REFUSED(ssm_conv1d_fwd_strided(4, 5120, 2048, 4, bf, 0, x, w, bias, s0, bf, y, hL, &cl, 0));
    ssm_conv_bld_layout_t cb = {0};
    cb.x_step = 5119;
    REFUSED(ssm_conv1d_fwd_bld(4, 5120, 2048, 4, bf, 0, x, w, bias, s0, bf, y, hL, &cb, 0));
    cb.x_step = 0;
    cb.y_batch = 1ll << 62;
    REFUSED(ssm_conv1d_fwd_bld(4, 5120, 2048, 4, bf, 0, x, w, bias, s0, bf, y, hL, &cb, 0));
    REFUSED(ssm_conv1d_fwd_bld(4, 5120, 2048, 4, bf, 0, x, w, bias, s0, bf, x, hL, 0, 0));
    REFUSED(ssm_conv1d_update(64, 5120, 1, bf, 0, s0, x, w, bias, bf, y, 0));
    REFUSED(ssm_conv1d_update_strided(64, 5120, 4, bf, 0, s0, x, w, bias, bf, y, -1, 0, 0));
    REFUSED(ssm_conv1d_update_strided(64, 5120, 4, bf, 0, s0, x, w, bias, bf, y, 0, 1ll << 62, 0));
    // backward
    void *dy = fake(15), *dx = fake(16), *ddt = fake(17), *dz = fake(18);
    float *dB = (float *)(fake(19)), *dC = (float *)(fake(20));
    float *dA = (float *)(fake(21)), *dD = (float *)(fake(22));
    float *dbias = (float *)(fake(23)), *dh0 = (float *)(fake(24));
    REFUSED(ssm_scan_bwd(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, NULL, dB, dC, dA, dD, dbias, dh0, ws, 1 << 20, 0));
    REFUSED(ssm_scan_bwd(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 4, 0));
    REFUSED(ssm_scan_bwd(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, dx, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 20, 0));
    REFUSED(ssm_scan_bwd(2, 8, 40, 16, bf, 8, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 20, 0));
    ssm_scan_bwd_layout_t bl = {0};
    bl.seq_batch[6] = -8;
    REFUSED(ssm_scan_bwd_strided(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 20, &bl, 0));
    bl.seq_batch[6] = 0;
    bl.bc_row = 1ll << 62;
    REFUSED(ssm_scan_bwd_strided(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 20, &bl, 0));
    // backward on (batch, L, dim) tensors
    sum += ssm_scan_bwd_bld_workspace_bytes(4, 5120, 2048, 16) + ssm_scan_bwd_bld_workspace_bytes(4, 5120, 2048, 3);
    ssm_scan_bwd_bld_layout_t bb;
    memset(&bb, 0, sizeof bb);
    bb.step[3] = 7;
    REFUSED(ssm_scan_bwd_bld(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 26, &bb, 0));
    bb.step[3] = 0;
    bb.C_batch = 1ll << 62;
    REFUSED(ssm_scan_bwd_bld(2, 8, 40, 16, bf, 0, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 26, &bb, 0));
    REFUSED(ssm_scan_bwd_bld(2, 8, 40, 16, bf, SSM_FLAG_CHECKPOINTS, x, dt, bias, A, Bm, Cm, Dk, z, h0, f32, dy, NULL, dx, ddt, dz, dB, dC, dA, dD, dbias, dh0, ws, 1 << 26, NULL, 0));

    printf("abi sanitizer run: %s (workspace checksum %zu)\n", failures ? "FAILED" : "ok", sum);
    return failures ? 1 : 0;
}
