/* Drives every entry point of include/moe.h through its validation and
 * dispatch code, for a host-only build of the C-ABI layer against
 * stub_launchers.cpp with AddressSanitizer and UndefinedBehaviorSanitizer
 * (test infrastructure).  The "device" buffers are host allocations that the
 * stub launchers never touch.  Checks that each rejected call returns the
 * documented code and launches nothing, and that accepted calls launch.
 * Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

extern long long stub_launches;

static int failures = 0;
#define EXPECT(call, code, launches)                                                                  \
    do {                                                                                            \
        long long before = stub_launches;                                                           \
        int rc = (call);                                                                            \
        int launched = stub_launches != before;                                                     \
        if (rc != (code) || launched != (launches)) {                                               \
            fprintf(stderr, "line %d: %s -> %d (want %d), launched %d\n", __LINE__, #call, rc, code, launched); \
            ++failures;                                                                             \
        }                                                                                           \
    } while (0)

static void* buf(size_t n)
{
    void* p = aligned_alloc(256, (n + 255) / 256 * 256);
    if (!p) exit(3);
    memset(p, 0, (n + 255) / 256 * 256);
    return p;
}

int main(void)
{
    const int T = 16, H = 256, E = 8, k = 2, I = 128, P = T * k;
    moe_dims d = {T, H, E, k, I, MOE_WFMT_BF16, MOE_PATH_AUTO};
    size_t ws_bytes = 0, ws_mx = 0;
    EXPECT(moe_workspace_size(&d, &ws_bytes), MOE_OK, 0);
    moe_dims dmx = d; dmx.wfmt = MOE_WFMT_MXFP4;
    EXPECT(moe_workspace_size(&dmx, &ws_mx), MOE_OK, 0);
    if (ws_mx <= ws_bytes) { fprintf(stderr, "the MX path's split activations add no workspace\n"); ++failures; }
    char* ws = buf(ws_mx);
    char* x = buf((size_t)T * H * 2);
    char* wr = buf((size_t)E * H * 2);
    char* gu = buf((size_t)E * 2 * I * H * 2);
    char* dn = buf((size_t)E * H * I * 2);
    uint8_t* sgu = buf((size_t)E * 2 * I * H / 32);
    uint8_t* sdn = buf((size_t)E * H * I / 32);
    char* y = buf((size_t)T * H * 2);
    int32_t* idx = buf((size_t)P * 4);
    float* w = buf((size_t)P * 4);
    int32_t* off = buf((size_t)(E + 1) * 4);
    int32_t* sp = buf((size_t)P * 4);
    int32_t* pr = buf((size_t)P * 4);
    char* h = buf((size_t)P * I * 2);
    char* ys = buf((size_t)P * H * 2);
    moe_expert_weights W = {gu, NULL, dn, NULL};
    moe_expert_weights WM = {gu, sgu, dn, sdn};

    /* dims validation */
    size_t n;
    EXPECT(moe_workspace_size(NULL, &n), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_workspace_size(&d, NULL), MOE_ERR_INVALID_ARG, 0);
    moe_dims bad = d; bad.T = -1; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_INVALID_ARG, 0);
    bad = d; bad.k = E + 1; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_INVALID_ARG, 0);
    bad = d; bad.k = 0; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_INVALID_ARG, 0);
    bad = d; bad.E = 257; bad.k = 2; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_UNSUPPORTED, 0);
    bad = d; bad.E = 16; bad.k = 9; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_UNSUPPORTED, 0);
    bad = d; bad.H = 48; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_UNSUPPORTED, 0);
    bad = d; bad.I = 40; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_UNSUPPORTED, 0);
    bad = d; bad.wfmt = 7; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_UNSUPPORTED, 0);
    bad = d; bad.path = 9; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_UNSUPPORTED, 0);
    bad = d; bad.T = 1 << 30; bad.k = 8; bad.E = 8; EXPECT(moe_workspace_size(&bad, &n), MOE_ERR_INVALID_ARG, 0);

    /* the fused layer, every schedule and format */
    for (int path = 0; path < 3; ++path)
        for (int fmt = 0; fmt < 3; ++fmt) {
            moe_dims dd = d;
            dd.path = path;
            dd.wfmt = fmt;
            EXPECT(moe_forward(&dd, x, wr, fmt ? &WM : &W, y, idx, w, ws, fmt ? ws_mx : ws_bytes, NULL), MOE_OK, 1);
        }
    /* the MX tiled path: MXFP4 only, H and I multiples of 64, its workspace */
    dmx.path = MOE_PATH_TILED_MX;
    EXPECT(moe_forward(&dmx, x, wr, &WM, y, NULL, NULL, ws, ws_mx, NULL), MOE_OK, 1);
    EXPECT(moe_forward(&dmx, x, wr, &WM, y, NULL, NULL, ws, ws_bytes, NULL), MOE_ERR_WORKSPACE, 0);
    EXPECT(moe_gate_up(&dmx, x, off, sp, &WM, h, ws, ws_bytes, NULL), MOE_ERR_WORKSPACE, 0);
    EXPECT(moe_gate_up(&dmx, x, off, sp, &WM, h, ws, ws_mx, NULL), MOE_OK, 1);
    EXPECT(moe_down(&dmx, h, off, &WM, ys, ws, ws_mx, NULL), MOE_OK, 1);
    moe_dims dbad = dmx; dbad.wfmt = MOE_WFMT_BF16;
    EXPECT(moe_workspace_size(&dbad, &n), MOE_ERR_UNSUPPORTED, 0);
    dbad = dmx; dbad.H = 96;
    EXPECT(moe_workspace_size(&dbad, &n), MOE_ERR_UNSUPPORTED, 0);
    dbad = dmx; dbad.path = 5;
    EXPECT(moe_workspace_size(&dbad, &n), MOE_ERR_UNSUPPORTED, 0);
    dbad = dmx; dbad.path = MOE_PATH_TILED_DEQUANT;
    EXPECT(moe_forward(&dbad, x, wr, &WM, y, NULL, NULL, ws, ws_mx, NULL), MOE_OK, 1);
    EXPECT(moe_mx_split(T, H, x, (uint8_t*)ys, sgu, NULL), MOE_OK, 1);
    EXPECT(moe_mx_split(T, 48, x, (uint8_t*)ys, sgu, NULL), MOE_ERR_UNSUPPORTED, 0);
    EXPECT(moe_mx_split(-1, H, x, (uint8_t*)ys, sgu, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_mx_split(T, H, x, (uint8_t*)ys + 8, sgu, NULL), MOE_ERR_MISALIGNED, 0);
    EXPECT(moe_mx_split(T, H, x, (uint8_t*)ys, sgu + 1, NULL), MOE_ERR_MISALIGNED, 0);
    EXPECT(moe_mx_split(0, H, NULL, NULL, NULL, NULL), MOE_OK, 0);
    EXPECT(moe_forward(&d, x, wr, &W, y, NULL, NULL, ws, ws_bytes, NULL), MOE_OK, 1);
    EXPECT(moe_forward(&d, NULL, wr, &W, y, NULL, NULL, ws, ws_bytes, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_forward(&d, x + 2, wr, &W, y, NULL, NULL, ws, ws_bytes, NULL), MOE_ERR_MISALIGNED, 0);
    EXPECT(moe_forward(&d, x, wr, &W, y, NULL, NULL, ws, ws_bytes - 1, NULL), MOE_ERR_WORKSPACE, 0);
    EXPECT(moe_forward(&d, x, wr, &W, y, idx, (float*)((char*)w + 2), ws, ws_bytes, NULL), MOE_ERR_MISALIGNED, 0);
    EXPECT(moe_forward(&d, x, wr, NULL, y, NULL, NULL, ws, ws_bytes, NULL), MOE_ERR_INVALID_ARG, 0);
    moe_dims dm = d; dm.wfmt = MOE_WFMT_MXFP4;
    EXPECT(moe_forward(&dm, x, wr, &W, y, NULL, NULL, ws, ws_mx, NULL), MOE_ERR_INVALID_ARG, 0);
    dm.wfmt = MOE_WFMT_MXFP4_PACKED;
    moe_expert_weights WP = {gu, sgu + 1, dn, sdn};
    EXPECT(moe_forward(&dm, x, wr, &WP, y, NULL, NULL, ws, ws_mx, NULL), MOE_ERR_MISALIGNED, 0);
    moe_dims d0 = d; d0.T = 0;
    EXPECT(moe_forward(&d0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK, 0);

    /* stages */
    EXPECT(moe_route(&d, x, wr, idx, w, ws, ws_bytes, NULL), MOE_OK, 1);
    EXPECT(moe_route(&d, x, wr, NULL, w, ws, ws_bytes, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_permute(&d, idx, off, sp, pr, ws, ws_bytes, NULL), MOE_OK, 1);
    EXPECT(moe_permute(&d, idx, off, sp, pr, ws, 16, NULL), MOE_ERR_WORKSPACE, 0);
    EXPECT(moe_gate_up(&d, x, off, sp, &W, h, ws, ws_bytes, NULL), MOE_OK, 1);
    EXPECT(moe_gate_up(&d, x, off, sp, &W, h + 8, ws, ws_bytes, NULL), MOE_ERR_MISALIGNED, 0);
    EXPECT(moe_down(&d, h, off, &W, ys, ws, ws_bytes, NULL), MOE_OK, 1);
    EXPECT(moe_down(&d, h, NULL, &W, ys, ws, ws_bytes, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_grouped_ffn(&d, x, off, sp, &W, ys, ws, ws_bytes, NULL), MOE_OK, 1);
    EXPECT(moe_grouped_ffn(&d, x, off, sp, &W, ys, ws, 0, NULL), MOE_ERR_WORKSPACE, 0);
    EXPECT(moe_combine(&d, ys, pr, w, y, NULL), MOE_OK, 1);
    EXPECT(moe_combine(&d, ys, pr, w, NULL, NULL), MOE_ERR_INVALID_ARG, 0);

    /* backward */
    size_t bws = 0;
    EXPECT(moe_backward_workspace_size(&d, &bws), MOE_OK, 0);
    EXPECT(moe_backward_workspace_size(&dm, &bws), MOE_ERR_UNSUPPORTED, 0);
    EXPECT(moe_backward_workspace_size(&d, &bws), MOE_OK, 0);
    char* bw = buf(bws);
    char* dx = buf((size_t)T * H * 2);
    float* dwr = buf((size_t)E * H * 4);
    float* dgu = buf((size_t)E * 2 * I * H * 4);
    float* ddn = buf((size_t)E * H * I * 4);
    EXPECT(moe_backward(&d, x, wr, &W, y, dx, dwr, dgu, ddn, bw, bws, NULL), MOE_OK, 1);
    EXPECT(moe_backward(&d, x, wr, &W, y, dx, dwr, dgu, ddn, bw, bws - 1, NULL), MOE_ERR_WORKSPACE, 0);
    EXPECT(moe_backward(&d, x, wr, &W, y, dx, NULL, dgu, ddn, bw, bws, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_backward(&d0, x, wr, &W, y, dx, dwr, dgu, ddn, bw, bws, NULL), MOE_OK, 1);

    /* quantiser and packed order */
    EXPECT(moe_mxfp4_quantize((int64_t)E * 2 * I, H, gu, (uint8_t*)h, sgu, NULL), MOE_OK, 1);
    EXPECT(moe_mxfp4_quantize(4, 40, gu, (uint8_t*)h, sgu, NULL), MOE_ERR_UNSUPPORTED, 0);
    EXPECT(moe_mxfp4_quantize(-1, 32, gu, (uint8_t*)h, sgu, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_mxfp4_quantize(0, 32, NULL, NULL, NULL, NULL), MOE_OK, 0);
    EXPECT(moe_mxfp4_quantize((int64_t)1 << 40, 64, gu, (uint8_t*)h, sgu, NULL), MOE_ERR_UNSUPPORTED, 0);
    EXPECT(moe_mxfp4_fakequant(8, 64, gu, ys, NULL), MOE_OK, 1);
    EXPECT(moe_mxfp4_fakequant(8, 64, gu, ys + 2, NULL), MOE_ERR_MISALIGNED, 0);
    uint8_t* wp = buf((size_t)E * 2 * I * H / 2);
    uint8_t* spk = buf((size_t)E * 2 * I * H / 32);
    EXPECT(moe_mxfp4_pack(&dm, MOE_PACK_GATE_UP, (uint8_t*)gu, sgu, wp, spk, NULL), MOE_OK, 1);
    EXPECT(moe_mxfp4_pack(&dm, MOE_PACK_DOWN, (uint8_t*)dn, sdn, wp, spk, NULL), MOE_OK, 1);
    EXPECT(moe_mxfp4_pack(&dm, 5, (uint8_t*)gu, sgu, wp, spk, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_mxfp4_pack(&dm, MOE_PACK_GATE_UP, (uint8_t*)gu, sgu, (uint8_t*)gu, spk, NULL), MOE_ERR_INVALID_ARG, 0);
    EXPECT(moe_mxfp4_pack(&dm, MOE_PACK_GATE_UP, (uint8_t*)gu, sgu, wp, spk + 4, NULL), MOE_ERR_MISALIGNED, 0);

    for (int c = -1; c <= 6; ++c)
        if (!moe_strerror(c) || !moe_strerror(c)[0]) { fprintf(stderr, "empty strerror(%d)\n", c); ++failures; }
    if (!moe_last_error()) ++failures;

    free(ws); free(x); free(wr); free(gu); free(dn); free(sgu); free(sdn); free(y); free(idx); free(w); free(off);
    free(sp); free(pr); free(h); free(ys); free(bw); free(dx); free(dwr); free(dgu); free(ddn); free(wp); free(spk);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
