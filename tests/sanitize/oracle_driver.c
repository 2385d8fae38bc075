/* Runs every entry point of the CPU oracle once on small seeded inputs, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure: checks the oracle's own memory and integer hygiene; the
 * values are checked elsewhere).  Prints "ok" and exits 0 when every call
 * returns success and its permutation outputs are consistent. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_route(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wr, double* logits, int32_t* topk_idx,
              double* topk_w, int threads);
int orc_permute(int T, int k, int E, const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_pairs,
                int32_t* pair_rank);
int orc_forward_tokens(int T, int H, int E, int k, int I, int wfmt, const uint16_t* x, const uint16_t* w_router,
                       const void* gate_up, const uint8_t* gate_up_scale, const void* down, const uint8_t* down_scale,
                       int n, const int32_t* tokens, double* y, int32_t* idx, double* w, double* o, double* h,
                       int threads);
int orc_backward(int T, int H, int E, int k, int I, const uint16_t* x, const uint16_t* w_router,
                 const uint16_t* gate_up, const uint16_t* down, const uint16_t* dy, double* dx, double* dw_router,
                 double* dgate_up, double* ddown, int threads);
int orc_mxfp4_quantize(int64_t rows, int64_t cols, const uint16_t* w, uint8_t* packed, uint8_t* scales);
int orc_mxfp4_fakequant(int64_t rows, int64_t cols, const uint16_t* w, uint16_t* out);
int orc_mxfp4_pack(int gate_up, int64_t E, int64_t I, int64_t H, const uint8_t* w, const uint8_t* s, uint8_t* wp,
                   uint8_t* sp);
int orc_mxfp4_unpack(int gate_up, int64_t E, int64_t I, int64_t H, const uint8_t* wp, const uint8_t* sp, uint8_t* w,
                     uint8_t* s);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) /* SplitMix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* a bf16 pattern of magnitude about 2^(e0 - 127 .. e0 - 124), random sign */
static uint16_t rand_bf16(int e0) { uint64_t r = next_u64(); return (uint16_t)(((r & 1) << 15) | ((e0 + (r >> 1) % 4) << 7) | ((r >> 8) & 0x7F)); }
static void* xalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) exit(3); return p; }

#define CHECK(call) do { if ((call) != 0) { fprintf(stderr, "failed: %s\n", #call); return 1; } } while (0)

int main(void)
{
    const int T = 9, H = 64, E = 5, k = 2, I = 96, P = T * k;
    uint16_t* x = xalloc(sizeof(uint16_t) * T * H);
    uint16_t* wr = xalloc(sizeof(uint16_t) * E * H);
    uint16_t* gu = xalloc(sizeof(uint16_t) * E * 2 * I * H);
    uint16_t* dn = xalloc(sizeof(uint16_t) * E * H * I);
    uint16_t* dy = xalloc(sizeof(uint16_t) * T * H);
    for (int i = 0; i < T * H; ++i) { x[i] = rand_bf16(127); dy[i] = rand_bf16(127); }
    for (int i = 0; i < E * H; ++i) wr[i] = rand_bf16(122);
    for (int i = 0; i < E * 2 * I * H; ++i) gu[i] = rand_bf16(120);
    for (int i = 0; i < E * H * I; ++i) dn[i] = rand_bf16(120);
    x[3 * H + 7] = 0x7FC0; /* a NaN token: its routing must still be k distinct experts */

    double* logits = xalloc(sizeof(double) * T * E);
    int32_t* idx = xalloc(sizeof(int32_t) * P);
    double* w = xalloc(sizeof(double) * P);
    CHECK(orc_route(T, H, E, k, x, wr, logits, idx, w, 1));
    int32_t* off = xalloc(sizeof(int32_t) * (E + 1));
    int32_t* sp = xalloc(sizeof(int32_t) * P);
    int32_t* pr = xalloc(sizeof(int32_t) * P);
    CHECK(orc_permute(T, k, E, idx, off, sp, pr));
    for (int p = 0; p < P; ++p)
        if (idx[p] < 0 || idx[p] >= E || sp[pr[p]] != p) { fprintf(stderr, "bad permutation at %d\n", p); return 1; }

    int32_t tokens[T];
    for (int t = 0; t < T; ++t) tokens[t] = t;
    double* y = xalloc(sizeof(double) * T * H);
    double* o = xalloc(sizeof(double) * P * H);
    double* h = xalloc(sizeof(double) * P * I);
    CHECK(orc_forward_tokens(T, H, E, k, I, 0, x, wr, gu, NULL, dn, NULL, T, tokens, y, idx, w, o, h, 1));

    /* MXFP4: quantise the bf16 weights, run the layer on them, pack and unpack */
    uint8_t* q_gu = xalloc((size_t)E * 2 * I * H / 2);
    uint8_t* s_gu = xalloc((size_t)E * 2 * I * H / 32);
    uint8_t* q_dn = xalloc((size_t)E * H * I / 2);
    uint8_t* s_dn = xalloc((size_t)E * H * I / 32);
    CHECK(orc_mxfp4_quantize((int64_t)E * 2 * I, H, gu, q_gu, s_gu));
    CHECK(orc_mxfp4_quantize((int64_t)E * H, I, dn, q_dn, s_dn));
    uint16_t* fq = xalloc(sizeof(uint16_t) * E * H * I);
    CHECK(orc_mxfp4_fakequant((int64_t)E * H, I, dn, fq));
    CHECK(orc_forward_tokens(T, H, E, k, I, 1, x, wr, q_gu, s_gu, q_dn, s_dn, T, tokens, y, idx, w, NULL, NULL, 1));
    uint8_t* wp = xalloc((size_t)E * 2 * I * H / 2);
    uint8_t* spk = xalloc((size_t)E * 2 * I * H / 32);
    uint8_t* wb = xalloc((size_t)E * 2 * I * H / 2);
    uint8_t* sb = xalloc((size_t)E * 2 * I * H / 32);
    CHECK(orc_mxfp4_pack(1, E, I, H, q_gu, s_gu, wp, spk));
    CHECK(orc_mxfp4_unpack(1, E, I, H, wp, spk, wb, sb));
    if (memcmp(wb, q_gu, (size_t)E * 2 * I * H / 2) || memcmp(sb, s_gu, (size_t)E * 2 * I * H / 32)) {
        fprintf(stderr, "pack/unpack round trip differs\n");
        return 1;
    }
    CHECK(orc_mxfp4_pack(0, E, I, H, q_dn, s_dn, wp, spk));
    CHECK(orc_mxfp4_unpack(0, E, I, H, wp, spk, wb, sb));

    double* dx = xalloc(sizeof(double) * T * H);
    double* dwr = xalloc(sizeof(double) * E * H);
    double* dgu = xalloc(sizeof(double) * E * 2 * I * H);
    double* ddn = xalloc(sizeof(double) * E * H * I);
    x[3 * H + 7] = 0x3F80; /* the backward takes finite inputs */
    CHECK(orc_backward(T, H, E, k, I, x, wr, gu, dn, dy, dx, dwr, dgu, ddn, 1));

    free(x); free(wr); free(gu); free(dn); free(dy); free(logits); free(idx); free(w); free(off); free(sp);
    free(pr); free(y); free(o); free(h); free(q_gu); free(s_gu); free(q_dn); free(s_dn); free(fq); free(wp);
    free(spk); free(wb); free(sb); free(dx); free(dwr); free(dgu); free(ddn);
    printf("ok\n");
    return 0;
}
