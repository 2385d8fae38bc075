/*
 * CPU oracle for the gpt-oss-style Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition the HIP library is checked against.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * path never does.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Every value is taken as the exact real number its bits encode and all
 * arithmetic is IEEE double in plain loop order, with no blocking, fusion or
 * intermediate rounding.
 *
 * What the layer computes, with sources:
 *  - top-4-of-32 (120b: of 128) expert routing per token and SwiGLU experts:
 *    "Persona Kappa: training a 20B LLM on desktop GPUs" (Level1Techs),
 *    table "Architecture Summary"; "hearth-lean-loomed-v1" model card,
 *    section "Why 12-16 streams can be slow on Vulkan".
 *  - expert weights natively MXFP4, activations kept in bf16 (W4A16):
 *    Persona Kappa post, section "Quantization-Aware Training (QAT)";
 *    "gpt-oss-20b" model page (coolboxapp), section "Architecture".
 *  The pages give no formulas.  The readings taken where they are silent:
 *    routing  = top-k by logit, ties to the lower expert index, slots in
 *               descending-logit order, softmax over the k selected;
 *    SwiGLU   = silu(gate) * up, silu(z) = z / (1 + exp(-z)), no bias/clamp;
 *    layouts  = weights stored [out][in] (K contiguous); the fused gate/up
 *               matrix has the I gate rows first, then the I up rows;
 *    MXFP4    = OCP Microscaling v1.0: E2M1 elements, one E8M0 scale per 32
 *               consecutive elements along K, element 2b in the low nibble
 *               of byte b and element 2b+1 in the high nibble;
 *    permute  = stable counting sort of pair ids p = t*k + j by expert.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NOMEM 2

/* Planted-mistake switch: the oracle's self-tests rebuild this file with
 * -DORC_PLANT=n to check that each pin catches a plausible mistake.  The
 * default build plants nothing. */
#ifndef ORC_PLANT
#define ORC_PLANT 0
#endif

/* ---------------------------------------------------------------- decode */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2:1 (bias 1), mantissa
 * bit 0.  Exponent field 0 is subnormal: 0.m * 2^0 = m/2. */
double orc_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0 scale: 2^(S-127); S = 255 encodes NaN. */
double orc_e8m0_value(unsigned s)
{
    if (s == 255u) return NAN;
    return ldexp(1.0, (int)s - 127);
}

/* Element c of an MXFP4 row: nibble c%2 of byte c/2, scaled by block c/32. */
double orc_mxfp4_value(const uint8_t* row_bytes, const uint8_t* row_scales, int64_t c)
{
    uint8_t b = row_bytes[c / 2];
#if ORC_PLANT == 5
    unsigned code = (c & 1) ? (b & 15u) : (b >> 4); /* planted: nibble order swapped */
#else
    unsigned code = (c & 1) ? (b >> 4) : (b & 15u);
#endif
    return orc_e2m1_value(code) * orc_e8m0_value(row_scales[c / 32]);
}

/* Decode matrix `expert` of a batched weight tensor [E][rows][cols] into
 * doubles.  wfmt 0: bf16 elements; wfmt 1: MXFP4 bytes [E][rows][cols/2] plus
 * scales [E][rows][cols/32]. */
static void decode_expert_matrix(int wfmt, const void* data, const uint8_t* scales,
                                 int64_t rows, int64_t cols, int64_t expert, double* out)
{
    for (int64_t r = 0; r < rows; ++r) {
        if (wfmt == 0) {
            const uint16_t* src = (const uint16_t*)data + (expert * rows + r) * cols;
            for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = orc_bf16_value(src[c]);
        } else {
            const uint8_t* rb = (const uint8_t*)data + (expert * rows + r) * (cols / 2);
            const uint8_t* rs = scales + (expert * rows + r) * (cols / 32);
            for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = orc_mxfp4_value(rb, rs, c);
        }
    }
}

int orc_decode_expert_matrix(int wfmt, const void* data, const uint8_t* scales,
                             int64_t rows, int64_t cols, int64_t expert, double* out)
{
    if (!data || !out || rows < 0 || cols < 0 || expert < 0) return ORC_ERR_ARG;
    if (wfmt == 1 && (!scales || cols % 32 != 0)) return ORC_ERR_ARG;
    if (wfmt != 0 && wfmt != 1) return ORC_ERR_ARG;
    decode_expert_matrix(wfmt, data, scales, rows, cols, expert, out);
    return ORC_OK;
}

/* ---------------------------------------------------------------- routing */

/* Router logit l[e] = sum_h x[h] * Wr[e][h], summed in h order. */
static void router_logits_one(int H, int E, const uint16_t* xrow, const uint16_t* wr, double* out)
{
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int h = 0; h < H; ++h)
            acc += orc_bf16_value(xrow[h]) * orc_bf16_value(wr[(int64_t)e * H + h]);
        out[e] = acc;
    }
}

/* The value a logit is ranked and weighted by.  The pages say nothing about
 * non-finite inputs; the reading taken: a NaN logit (a NaN in the token's
 * row or in the expert's router row) ranks below every number, as -infinity,
 * so selection always yields k distinct experts.  A token whose logits are
 * all NaN gets experts 0..k-1 by the tie rule, and NaN weights. */
static double rank_key(double v)
{
#if ORC_PLANT == 8
    return v; /* planted: NaN logits compared raw */
#else
    return isnan(v) ? -INFINITY : v;
#endif
}

/* Does expert a come before expert b in routing order?  Larger logit first;
 * an exactly equal logit puts the lower index first. */
static int route_before(const double* l, int a, int b)
{
    const double la = rank_key(l[a]), lb = rank_key(l[b]);
#if ORC_PLANT == 2
    if (la == lb) return a > b; /* planted: ties go to the higher index */
#else
    if (la == lb) return a < b;
#endif
    return la > lb;
}

/* Order all E experts by routing order (insertion sort), keep the first k as
 * the slots, and weight them by a softmax over the k selected logits. */
static void select_topk_one(int E, int k, const double* l, int32_t* idx, double* w, int* order)
{
    for (int e = 0; e < E; ++e) {
        int pos = e;
        while (pos > 0 && route_before(l, e, order[pos - 1])) {
            order[pos] = order[pos - 1];
            --pos;
        }
        order[pos] = e;
    }
    double lmax = rank_key(l[order[0]]);
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(rank_key(l[order[j]]) - lmax);
    for (int j = 0; j < k; ++j) {
        idx[j] = order[j];
#if ORC_PLANT == 7
        w[j] = exp(rank_key(l[order[j]]) - lmax); /* planted: weights not normalised */
#else
        w[j] = exp(rank_key(l[order[j]]) - lmax) / z;
#endif
    }
}

/* Route T tokens: logits [T][E] (optional), topk_idx [T][k], topk_w [T][k]. */
int orc_route(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wr,
              double* logits, int32_t* topk_idx, double* topk_w, int threads)
{
    if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || !x || !wr || !topk_idx || !topk_w)
        return ORC_ERR_ARG;
    int err = ORC_OK;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double* l = (double*)malloc(sizeof(double) * (size_t)E);
        int* order = (int*)malloc(sizeof(int) * (size_t)E);
        if (!l || !order) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        }
        /* every thread reaches the work-sharing loop; one without buffers skips its share */
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            if (!l || !order) continue;
            router_logits_one(H, E, x + (int64_t)t * H, wr, l);
            if (logits) memcpy(logits + (int64_t)t * E, l, sizeof(double) * (size_t)E);
            select_topk_one(E, k, l, topk_idx + (int64_t)t * k, topk_w + (int64_t)t * k, order);
        }
        free(l);
        free(order);
    }
    return err;
}

/* ---------------------------------------------------------------- permute */

/* Stable counting sort of the P = T*k pair ids by expert.
 * expert_offsets [E+1]: exclusive prefix sum of the per-expert counts.
 * sorted_pairs [P]: pair ids in expert-major order, ascending p inside each
 * expert.  pair_rank [P]: the inverse, pair_rank[sorted_pairs[s]] = s. */
int orc_permute(int T, int k, int E, const int32_t* topk_idx,
                int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_rank)
{
    if (T < 0 || k < 1 || E <= 0 || !topk_idx || !expert_offsets || (T > 0 && (!sorted_pairs || !pair_rank)))
        return ORC_ERR_ARG;
    int64_t P = (int64_t)T * k;
    int32_t* cursor = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!cursor) return ORC_ERR_NOMEM;
    for (int e = 0; e <= E; ++e) expert_offsets[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = topk_idx[p];
        if (e < 0 || e >= E) {
            free(cursor);
            return ORC_ERR_ARG;
        }
        expert_offsets[e + 1] += 1;
    }
    for (int e = 0; e < E; ++e) expert_offsets[e + 1] += expert_offsets[e];
    for (int e = 0; e < E; ++e) cursor[e] = expert_offsets[e];
#if ORC_PLANT == 4
    for (int64_t p = P - 1; p >= 0; --p) { /* planted: not stable */
#else
    for (int64_t p = 0; p < P; ++p) {
#endif
        int32_t e = topk_idx[p];
        int32_t s = cursor[e]++;
        sorted_pairs[s] = (int32_t)p;
        pair_rank[p] = s;
    }
    free(cursor);
    return ORC_OK;
}

/* ---------------------------------------------------------------- experts */

static double silu(double z)
{
#if ORC_PLANT == 6
    return z / (1.0 + exp(z)); /* planted: sign error */
#else
    return z / (1.0 + exp(-z));
#endif
}

/* One expert on one token, with the expert's weights already decoded:
 *   g_i = sum_h x_h Wgu[i][h],  u_i = sum_h x_h Wgu[I+i][h]   (i < I)
 *   a_i = silu(g_i) * u_i
 *   o_n = sum_i a_i Wd[n][i]                                  (n < H)
 * h_out (I values) is optional. */
static void expert_ffn_one(int H, int I, const double* xrow, const double* wgu, const double* wd,
                           double* a, double* h_out, double* o_out)
{
    for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
#if ORC_PLANT == 1
        const double* grow = wgu + (int64_t)(I + i) * H; /* planted: gate and up swapped */
        const double* urow = wgu + (int64_t)i * H;
#else
        const double* grow = wgu + (int64_t)i * H;
        const double* urow = wgu + (int64_t)(I + i) * H;
#endif
        for (int h = 0; h < H; ++h) g += xrow[h] * grow[h];
        for (int h = 0; h < H; ++h) u += xrow[h] * urow[h];
        a[i] = silu(g) * u;
        if (h_out) h_out[i] = a[i];
    }
    for (int n = 0; n < H; ++n) {
        double acc = 0.0;
#if ORC_PLANT == 3
        for (int i = 0; i < I; ++i) acc += a[i] * wd[(int64_t)i * H + n]; /* planted: Wd read transposed */
#else
        for (int i = 0; i < I; ++i) acc += a[i] * wd[(int64_t)n * I + i];
#endif
        o_out[n] = acc;
    }
}

/* Expert outputs for a list of (token, expert) pairs.
 * x bf16 [T][H]; gate_up [E][2I][H] (bf16) or [E][2I][H/2] + scales
 * [E][2I][H/32] (MXFP4); down [E][H][I] or [E][H][I/2] + [E][H][I/32].
 * h_out [npairs][I] (optional, SwiGLU output), o_out [npairs][H].
 * Work is grouped by expert so each expert's weights are decoded once. */
int orc_ffn_pairs(int H, int I, int E, int wfmt, const uint16_t* x,
                  const void* gate_up, const uint8_t* gate_up_scale,
                  const void* down, const uint8_t* down_scale,
                  int npairs, const int32_t* pair_token, const int32_t* pair_expert,
                  double* h_out, double* o_out, int threads)
{
    if (H <= 0 || I <= 0 || E <= 0 || npairs < 0 || !x || !gate_up || !down || !o_out ||
        (npairs > 0 && (!pair_token || !pair_expert)))
        return ORC_ERR_ARG;
    if (wfmt != 0 && wfmt != 1) return ORC_ERR_ARG;
    if (wfmt == 1 && (!gate_up_scale || !down_scale || H % 32 || I % 32)) return ORC_ERR_ARG;
    for (int q = 0; q < npairs; ++q)
        if (pair_expert[q] < 0 || pair_expert[q] >= E || pair_token[q] < 0) return ORC_ERR_ARG;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    double* wgu = (double*)malloc(sizeof(double) * (size_t)2 * I * H);
    double* wd = (double*)malloc(sizeof(double) * (size_t)H * I);
    int32_t* list = (int32_t*)malloc(sizeof(int32_t) * (size_t)(npairs > 0 ? npairs : 1));
    if (!wgu || !wd || !list) {
        free(wgu);
        free(wd);
        free(list);
        return ORC_ERR_NOMEM;
    }
    int err = ORC_OK;
    for (int e = 0; e < E && err == ORC_OK; ++e) {
        int n = 0;
        for (int q = 0; q < npairs; ++q)
            if (pair_expert[q] == e) list[n++] = q;
        if (n == 0) continue;
        decode_expert_matrix(wfmt, gate_up, gate_up_scale, 2 * (int64_t)I, H, e, wgu);
        decode_expert_matrix(wfmt, down, down_scale, H, I, e, wd);
#pragma omp parallel
        {
            double* xr = (double*)malloc(sizeof(double) * (size_t)H);
            double* a = (double*)malloc(sizeof(double) * (size_t)I);
            if (!xr || !a) {
#pragma omp atomic write
                err = ORC_ERR_NOMEM;
            }
#pragma omp for schedule(dynamic, 1)
            for (int j = 0; j < n; ++j) {
                if (!xr || !a) continue;
                int q = list[j];
                const uint16_t* xs = x + (int64_t)pair_token[q] * H;
                for (int h = 0; h < H; ++h) xr[h] = orc_bf16_value(xs[h]);
                expert_ffn_one(H, I, xr, wgu, wd, a, h_out ? h_out + (int64_t)q * I : NULL,
                               o_out + (int64_t)q * H);
            }
            free(xr);
            free(a);
        }
    }
    free(wgu);
    free(wd);
    free(list);
    return err;
}

/* ---------------------------------------------------------------- layer */

/* Whole layer for a subset of tokens (each token's output depends on that
 * token alone):  y[t] = sum_j w[t][j] * expert_{idx[t][j]}(x[t]), the k terms
 * added in slot order.  tokens [ntok] are row indices into x; y_out
 * [ntok][H].  Optional: idx_out [ntok][k], w_out [ntok][k], the per-slot
 * expert outputs o_out [ntok][k][H] and SwiGLU activations h_out [ntok][k][I]. */
int orc_forward_tokens(int T, int H, int E, int k, int I, int wfmt,
                       const uint16_t* x, const uint16_t* w_router,
                       const void* gate_up, const uint8_t* gate_up_scale,
                       const void* down, const uint8_t* down_scale,
                       int ntok, const int32_t* tokens,
                       double* y_out, int32_t* idx_out, double* w_out,
                       double* o_out, double* h_out, int threads)
{
    if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || I <= 0 || ntok < 0 || !x || !w_router || !y_out ||
        (ntok > 0 && !tokens))
        return ORC_ERR_ARG;
    for (int i = 0; i < ntok; ++i)
        if (tokens[i] < 0 || tokens[i] >= T) return ORC_ERR_ARG;
    size_t nk = (size_t)(ntok > 0 ? ntok : 1) * (size_t)k;
    uint16_t* xs = (uint16_t*)calloc((size_t)(ntok > 0 ? ntok : 1) * (size_t)H, sizeof(uint16_t));
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * nk);
    double* w = (double*)malloc(sizeof(double) * nk);
    int32_t* ptok = (int32_t*)malloc(sizeof(int32_t) * nk);
    double* o = (double*)malloc(sizeof(double) * nk * (size_t)H);
    int err = ORC_ERR_NOMEM;
    if (xs && idx && w && ptok && o) {
        for (int i = 0; i < ntok; ++i) memcpy(xs + (int64_t)i * H, x + (int64_t)tokens[i] * H, sizeof(uint16_t) * H);
        err = orc_route(ntok, H, E, k, xs, w_router, NULL, idx, w, threads);
        if (err == ORC_OK) {
            for (int i = 0; i < ntok; ++i)
                for (int j = 0; j < k; ++j) ptok[i * k + j] = i;
            err = orc_ffn_pairs(H, I, E, wfmt, xs, gate_up, gate_up_scale, down, down_scale, ntok * k, ptok, idx,
                                h_out, o, threads);
        }
        if (err == ORC_OK) {
            for (int i = 0; i < ntok; ++i)
                for (int n = 0; n < H; ++n) {
                    double acc = 0.0;
                    for (int j = 0; j < k; ++j) acc += w[i * k + j] * o[((int64_t)i * k + j) * H + n];
                    y_out[(int64_t)i * H + n] = acc;
                }
            if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)ntok * k);
            if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)ntok * k);
            if (o_out) memcpy(o_out, o, sizeof(double) * (size_t)ntok * k * H);
        }
    }
    free(xs);
    free(idx);
    free(w);
    free(ptok);
    free(o);
    return err;
}

/* ---------------------------------------------------------- backward */

/* Gradients of the layer (the training variant: the pages fine-tune every
 * expert's parameters in bf16 with fp32 reductions, "Persona Kappa: training
 * a 20B LLM on desktop GPUs", section "Techniques That Made It Fit"), for the
 * loss L = sum_t dy[t] . y[t], i.e. the backward pass given the upstream
 * gradient dy.  The selection of the k experts is piecewise constant in the
 * logits, so gradients flow only through the k selected softmax weights.
 * Per slot j of token t with expert e (forward as above):
 *   dw_j   = dy . o_j
 *   do_j   = w_j dy
 *   da     = Wd^T do_j                     dWd[e]  += do_j a^T
 *   dg     = da * u * silu'(g)             silu'(z) = s(z) (1 + z (1 - s(z))),  s = logistic
 *   du     = da * silu(g)                  dWgu[e] += [dg; du] x^T
 *   dx    += Wg^T dg + Wu^T du
 * and per token, through the softmax over the k selected logits:
 *   dl_j   = w_j (dw_j - sum_i w_i dw_i)
 *   dx    += sum_j dl_j Wr[e_j]             dWr[e_j] += dl_j x
 * All in double, from the exact input values. */

static double logistic(double z) { return 1.0 / (1.0 + exp(-z)); }

static double silu_grad(double z)
{
    double s = logistic(z);
#if ORC_PLANT == 30
    return s; /* planted: the z s (1 - s) term dropped */
#else
    return s * (1.0 + z * (1.0 - s));
#endif
}

/* Source of one expert's weights as doubles: bf16 bit patterns decoded, or
 * double arrays used in place. */
typedef struct {
    const uint16_t* gate_up_bf16;
    const uint16_t* down_bf16;
    const double* gate_up_f64;
    const double* down_f64;
} weights_src;

static void expert_weights_f64(const weights_src* src, int H, int I, int e, double* wgu, double* wd)
{
    const int64_t ngu = 2 * (int64_t)I * H, nd = (int64_t)H * I;
    if (src->gate_up_f64) {
        memcpy(wgu, src->gate_up_f64 + e * ngu, sizeof(double) * (size_t)ngu);
        memcpy(wd, src->down_f64 + e * nd, sizeof(double) * (size_t)nd);
    } else {
        for (int64_t i = 0; i < ngu; ++i) wgu[i] = orc_bf16_value(src->gate_up_bf16[e * ngu + i]);
        for (int64_t i = 0; i < nd; ++i) wd[i] = orc_bf16_value(src->down_bf16[e * nd + i]);
    }
}

/* The backward of T tokens.  x, dy [T][H] and wr [E][H] as doubles; outputs
 * (all overwritten): dx [T][H], dwr [E][H], dgu [E][2I][H], ddn [E][H][I];
 * optional: loss (sum dy . y), idx_out [T][k]. */
static int backward_core(int T, int H, int E, int k, int I, const double* x, const double* wr,
                         const weights_src* src, const double* dy, double* dx, double* dwr, double* dgu,
                         double* ddn, double* loss, int32_t* idx_out)
{
    const size_t Tk = (size_t)(T > 0 ? T : 1) * (size_t)k;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * Tk);
    double* w = (double*)malloc(sizeof(double) * Tk);
    double* dw = (double*)calloc(Tk, sizeof(double));
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
    double* wgu = (double*)malloc(sizeof(double) * (size_t)2 * I * H);
    double* wd = (double*)malloc(sizeof(double) * (size_t)H * I);
    int32_t* list = (int32_t*)malloc(sizeof(int32_t) * Tk);
    /* per pair of the current expert: a, do, and [dg; du] */
    double *pa = NULL, *pdo = NULL, *pdgu = NULL;
    int err = ORC_ERR_NOMEM;
    if (!idx || !w || !dw || !lg || !order || !wgu || !wd || !list) goto done;
    memset(dx, 0, sizeof(double) * (size_t)T * H);
    memset(dwr, 0, sizeof(double) * (size_t)E * H);
    memset(dgu, 0, sizeof(double) * (size_t)E * 2 * I * H);
    memset(ddn, 0, sizeof(double) * (size_t)E * H * I);
    /* routing */
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += x[(int64_t)t * H + h] * wr[(int64_t)e * H + h];
            lg[e] = acc;
        }
        select_topk_one(E, k, lg, idx + (size_t)t * k, w + (size_t)t * k, order);
    }
    double total = 0.0;
    for (int e = 0; e < E; ++e) {
        int n = 0;
        for (int q = 0; q < T * k; ++q)
            if (idx[q] == e) list[n++] = q;
        if (n == 0) continue;
        expert_weights_f64(src, H, I, e, wgu, wd);
        free(pa);
        free(pdo);
        free(pdgu);
        pa = (double*)malloc(sizeof(double) * (size_t)n * I);
        pdo = (double*)malloc(sizeof(double) * (size_t)n * H);
        pdgu = (double*)malloc(sizeof(double) * (size_t)n * 2 * I);
        if (!pa || !pdo || !pdgu) goto done;
        double part = 0.0;
        /* per pair: forward, dw, do, da, [dg; du], dx (a token occurs at most
         * once per expert, so the dx rows of one expert's pairs are distinct) */
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : part)
        for (int j = 0; j < n; ++j) {
            const int q = list[j], t = q / k;
            const double* xr = x + (int64_t)t * H;
            const double* dyr = dy + (int64_t)t * H;
            double* g = (double*)malloc(sizeof(double) * (size_t)2 * I); /* g then u */
            double* da = (double*)malloc(sizeof(double) * (size_t)I);
            if (!g || !da) {
                free(g);
                free(da);
                continue;
            }
            double* a = pa + (int64_t)j * I;
            double* dor = pdo + (int64_t)j * H;
            double* dgur = pdgu + (int64_t)j * 2 * I;
            for (int r = 0; r < 2 * I; ++r) {
                double acc = 0.0;
                for (int h = 0; h < H; ++h) acc += xr[h] * wgu[(int64_t)r * H + h];
                g[r] = acc;
            }
            for (int i = 0; i < I; ++i) a[i] = silu(g[i]) * g[I + i];
            double dwq = 0.0;
            for (int nn = 0; nn < H; ++nn) {
                double o = 0.0;
                for (int i = 0; i < I; ++i) o += a[i] * wd[(int64_t)nn * I + i];
                dwq += dyr[nn] * o;
            }
            dw[q] = dwq;
            part += w[q] * dwq;
            for (int nn = 0; nn < H; ++nn) dor[nn] = w[q] * dyr[nn];
            for (int i = 0; i < I; ++i) {
                double acc = 0.0;
                for (int nn = 0; nn < H; ++nn) acc += dor[nn] * wd[(int64_t)nn * I + i];
                da[i] = acc;
            }
            for (int i = 0; i < I; ++i) {
                dgur[i] = da[i] * g[I + i] * silu_grad(g[i]);
                dgur[I + i] = da[i] * silu(g[i]);
            }
            double* dxr = dx + (int64_t)t * H;
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int r = 0; r < 2 * I; ++r) acc += dgur[r] * wgu[(int64_t)r * H + h];
                dxr[h] += acc;
            }
            free(g);
            free(da);
        }
        total += part;
        /* weight gradients, summed over the expert's pairs in list order */
        double* dde = ddn + (int64_t)e * H * I;
#pragma omp parallel for schedule(static)
        for (int nn = 0; nn < H; ++nn)
            for (int i = 0; i < I; ++i) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += pdo[(int64_t)j * H + nn] * pa[(int64_t)j * I + i];
#if ORC_PLANT == 31
                dde[(int64_t)i * H + nn % I] = acc; /* planted: written transposed (square case) */
#else
                dde[(int64_t)nn * I + i] = acc;
#endif
            }
        double* dge = dgu + (int64_t)e * 2 * I * H;
#pragma omp parallel for schedule(static)
        for (int r = 0; r < 2 * I; ++r)
            for (int h = 0; h < H; ++h) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += pdgu[(int64_t)j * 2 * I + r] * x[(int64_t)(list[j] / k) * H + h];
                dge[(int64_t)r * H + h] = acc;
            }
    }
    /* router, through the softmax over the k selected logits */
    for (int t = 0; t < T; ++t) {
        double sbar = 0.0;
        for (int j = 0; j < k; ++j) sbar += w[(size_t)t * k + j] * dw[(size_t)t * k + j];
        for (int j = 0; j < k; ++j) {
            const size_t q = (size_t)t * k + j;
#if ORC_PLANT == 32
            const double dl = w[q] * dw[q]; /* planted: the mean term dropped */
#else
            const double dl = w[q] * (dw[q] - sbar);
#endif
            const int e = idx[q];
            for (int h = 0; h < H; ++h) {
                dx[(int64_t)t * H + h] += dl * wr[(int64_t)e * H + h];
                dwr[(int64_t)e * H + h] += dl * x[(int64_t)t * H + h];
            }
        }
    }
    if (loss) *loss = total;
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)T * k);
    err = ORC_OK;
done:
    free(idx);
    free(w);
    free(dw);
    free(lg);
    free(order);
    free(wgu);
    free(wd);
    free(list);
    free(pa);
    free(pdo);
    free(pdgu);
    return err;
}

static int backward_args_ok(int T, int H, int E, int k, int I)
{
    return T >= 0 && H > 0 && E > 0 && k >= 1 && k <= E && I > 0;
}

/* bf16 inputs (x, dy [T][H]; w_router [E][H]; gate_up [E][2I][H]; down
 * [E][H][I]) -> double gradients dx [T][H], dw_router [E][H], dgate_up
 * [E][2I][H], ddown [E][H][I]. */
int orc_backward(int T, int H, int E, int k, int I, const uint16_t* x, const uint16_t* w_router,
                 const uint16_t* gate_up, const uint16_t* down, const uint16_t* dy, double* dx, double* dw_router,
                 double* dgate_up, double* ddown, int threads)
{
    if (!backward_args_ok(T, H, E, k, I) || !x || !w_router || !gate_up || !down || !dy || !dx || !dw_router ||
        !dgate_up || !ddown)
        return ORC_ERR_ARG;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
    const size_t nx = (size_t)(T > 0 ? T : 1) * H;
    double* xd = (double*)malloc(sizeof(double) * nx);
    double* dyd = (double*)malloc(sizeof(double) * nx);
    double* wrd = (double*)malloc(sizeof(double) * (size_t)E * H);
    int err = ORC_ERR_NOMEM;
    if (xd && dyd && wrd) {
        for (size_t i = 0; i < (size_t)T * H; ++i) {
            xd[i] = orc_bf16_value(x[i]);
            dyd[i] = orc_bf16_value(dy[i]);
        }
        for (size_t i = 0; i < (size_t)E * H; ++i) wrd[i] = orc_bf16_value(w_router[i]);
        weights_src src = {gate_up, down, NULL, NULL};
        err = backward_core(T, H, E, k, I, xd, wrd, &src, dyd, dx, dw_router, dgate_up, ddown, NULL, NULL);
    }
    free(xd);
    free(dyd);
    free(wrd);
    return err;
}

/* The same on double inputs (for finite-difference checks), also returning
 * the loss sum_t dy[t] . y[t] and the routing. */
int orc_backward_f64(int T, int H, int E, int k, int I, const double* x, const double* w_router,
                     const double* gate_up, const double* down, const double* dy, double* dx, double* dw_router,
                     double* dgate_up, double* ddown, double* loss, int32_t* idx_out)
{
    if (!backward_args_ok(T, H, E, k, I) || !x || !w_router || !gate_up || !down || !dy || !dx || !dw_router ||
        !dgate_up || !ddown)
        return ORC_ERR_ARG;
    weights_src src = {NULL, NULL, gate_up, down};
    return backward_core(T, H, E, k, I, x, w_router, &src, dy, dx, dw_router, dgate_up, ddown, loss, idx_out);
}

/* ---------------------------------------------------------- quantize */

/* MXFP4 quantizer: the step that produces the experts' MXFP4 weights from
 * bf16 ones (the QAT run trains through fake-quantised expert weights and
 * then exports them quantised: "Persona Kappa: training a 20B LLM on desktop
 * GPUs", section "Quantization-Aware Training (QAT)").  The pages do not
 * print the rounding rule; this is the OCP Microscaling v1.0 one:
 *   per block of 32 consecutive elements along a row, with amax = max |v|,
 *   X = floor(log2 amax) - 2 (2 is the exponent of the largest E2M1
 *   magnitude, 6 = 1.5 * 2^2) and the E8M0 byte S = clamp(X + 127, 0, 254);
 *   an all-zero block stores S = 0 and zero codes;
 *   each element v / 2^(S-127) goes to the nearest E2M1 magnitude (values
 *   beyond 6 to 6), an exact midpoint to the even code; the sign bit is set
 *   only on a nonzero code of a negative element. */

/* Nearest of the eight E2M1 magnitudes to mag >= 0; on an exact tie the
 * even code.  The magnitudes and mag are exact in double, so are the
 * distances. */
static unsigned e2m1_nearest(double mag)
{
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c < 8; ++c) {
        double d = fabs(orc_e2m1_value(c) - mag);
#if ORC_PLANT == 20
        int take = d < bestd || (d == bestd && (c % 2 == 1)); /* planted: ties to the odd code */
#else
        int take = d < bestd || (d == bestd && (c % 2 == 0));
#endif
        if (take) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* Quantise one block of 32 bf16 values: 32 codes (low nibble = element 0 of
 * a pair) and the scale byte. */
static void quantize_block(const uint16_t* v, uint8_t codes[32], uint8_t* scale)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(orc_bf16_value(v[i])));
    unsigned S = 0;
    if (amax > 0.0) {
        int e;
        frexp(amax, &e); /* amax = m * 2^e, m in [0.5, 1): floor(log2 amax) = e - 1 */
#if ORC_PLANT == 21
        int X = (e - 1) - 1; /* planted: one octave too high */
#else
        int X = (e - 1) - 2;
#endif
        int s = X + 127;
        S = s < 0 ? 0u : (s > 254 ? 254u : (unsigned)s);
    }
    double unit = ldexp(1.0, (int)S - 127);
    for (int i = 0; i < 32; ++i) {
        double x = orc_bf16_value(v[i]);
        unsigned c = amax > 0.0 ? e2m1_nearest(fabs(x) / unit) : 0u;
#if ORC_PLANT == 22
        if (x < 0.0 || signbit(x)) c |= 8u; /* planted: negative zero kept */
#else
        if (x < 0.0 && c != 0u) c |= 8u;
#endif
        codes[i] = (uint8_t)c;
    }
    *scale = (uint8_t)S;
}

/* w bf16 [rows][cols] -> packed u8 [rows][cols/2] (element 2b in the low
 * nibble of byte b) and scales u8 [rows][cols/32].  cols % 32 == 0. */
int orc_mxfp4_quantize(int64_t rows, int64_t cols, const uint16_t* w, uint8_t* packed, uint8_t* scales)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0 || (rows * cols > 0 && (!w || !packed || !scales))) return ORC_ERR_ARG;
    const int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t codes[32];
            quantize_block(w + r * cols + 32 * b, codes, scales + r * nb + b);
            uint8_t* out = packed + r * (cols / 2) + 16 * b;
            for (int i = 0; i < 16; ++i) out[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
        }
    return ORC_OK;
}

/* Fake quantisation: w -> decode(quantize(w)) as bf16 [rows][cols].  Every
 * decoded value (at most two significant bits, exponent within bf16's range
 * since S <= 252 for finite bf16 input) is exactly a bf16 value, so the
 * conversion below does not round; it fails if it would. */
int orc_mxfp4_fakequant(int64_t rows, int64_t cols, const uint16_t* w, uint16_t* out)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0 || (rows * cols > 0 && (!w || !out))) return ORC_ERR_ARG;
    const int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t codes[32], S, bytes[16];
            quantize_block(w + r * cols + 32 * b, codes, &S);
            for (int i = 0; i < 16; ++i) bytes[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
            for (int i = 0; i < 32; ++i) {
                double v = orc_mxfp4_value(bytes, &S, i);
                float f = (float)v;
                uint32_t u;
                memcpy(&u, &f, sizeof u);
                if ((double)f != v || (u & 0xFFFFu) != 0u) return ORC_ERR_ARG;
                out[r * cols + 32 * b + i] = (uint16_t)(u >> 16);
            }
        }
    return ORC_OK;
}

/* ------------------------------------------------------- packed MXFP4 order
 *
 * A storage order for MXFP4 expert weights that this library defines for
 * decode-time weight streaming.  The pages fix the number format (E2M1 + one
 * E8M0 scale per 32 elements, "Persona Kappa" post, section "Quantization-
 * Aware Training (QAT)"), not a byte order; this order keeps every byte and
 * scale unchanged and only moves them.  Per expert, a piece is the 16 bytes
 * of one row over one K-block (elements 32kb .. 32kb+31 of the row), and it
 * carries that block's scale byte.  Rows form items of 32 slots:
 *   gate/up tensor [2I][K=H]: item i has gate rows 16i..16i+15 in slots
 *                              0..15 and up rows I+16i..I+16i+15 in 16..31;
 *   down tensor [H][K=I]:     item i has rows 32i..32i+31 in slots 0..31.
 * Write slot q = 4g + t (g < 8, t < 4) and K-block kb = 16c + b (chunk c,
 * b < 16); with nkb = K/32 and nb(c) = min(16, nkb - 16c) blocks in chunk c,
 * the piece (item i, slot q, kb) sits at byte
 *     i*512*nkb + c*8192 + g*64*nb(c) + 16*(4b + t)
 * of the expert's packed bytes and its scale at byte
 *     i*32*nkb + c*512 + 8*(4b + t) + g
 * of the expert's packed scales.  Experts follow each other at the same
 * strides as in the row-major layout (rows*K/2 bytes, rows*K/32 scales).
 *
 * orc_mxfp4_pack computes each piece's destination from the formula above;
 * orc_mxfp4_unpack walks the packed bytes in address order (item, chunk,
 * then g, b, t for bytes and b, t, g for scales) and derives each source
 * from the loop position, so the two are independent descriptions of one
 * permutation. */

/* Row of expert-local slot q of item i (gate_up != 0: paired gate/up rows). */
static int64_t packed_slot_row(int gate_up, int64_t I, int64_t i, int q)
{
    if (!gate_up) return 32 * i + q;
#if ORC_PLANT == 40
    return 16 * i + q; /* planted: up rows read from the gate half */
#else
    return q < 16 ? 16 * i + q : I + 16 * i + (q - 16);
#endif
}

static int packed_args_ok(int gate_up, int64_t E, int64_t I, int64_t H)
{
    /* items of 32 rows (gate/up pairs 16 columns of each half) and whole K-blocks */
    if (E <= 0 || I <= 0 || H <= 0 || (gate_up != 0 && gate_up != 1)) return 0;
    return gate_up ? I % 16 == 0 && H % 32 == 0 : H % 32 == 0 && I % 32 == 0;
}

/* gate_up = 1: w u8 [E][2I][H/2], s u8 [E][2I][H/32]; gate_up = 0: w u8
 * [E][H][I/2], s u8 [E][H][I/32].  Writes wp, sp of the same sizes. */
int orc_mxfp4_pack(int gate_up, int64_t E, int64_t I, int64_t H, const uint8_t* w, const uint8_t* s, uint8_t* wp,
                   uint8_t* sp)
{
    if (!packed_args_ok(gate_up, E, I, H) || !w || !s || !wp || !sp) return ORC_ERR_ARG;
    const int64_t R = gate_up ? 2 * I : H, K = gate_up ? H : I, nkb = K / 32;
    for (int64_t e = 0; e < E; ++e) {
        const uint8_t* we = w + e * R * (K / 2);
        const uint8_t* se = s + e * R * nkb;
        uint8_t* wpe = wp + e * R * (K / 2);
        uint8_t* spe = sp + e * R * nkb;
        for (int64_t r = 0; r < R; ++r) {
            int64_t i;
            int q;
            if (gate_up) {
                const int64_t n = r < I ? r : r - I; /* output column of the row */
                i = n / 16;
                q = (int)(n % 16) + (r < I ? 0 : 16);
            } else {
                i = r / 32;
                q = (int)(r % 32);
            }
            const int g = q / 4, t = q % 4;
            for (int64_t kb = 0; kb < nkb; ++kb) {
                const int64_t c = kb / 16, b = kb % 16;
                const int64_t nb = nkb - 16 * c < 16 ? nkb - 16 * c : 16;
#if ORC_PLANT == 41
                const int64_t dst = i * 512 * nkb + c * 512 * nb + g * 64 * nb + 16 * (4 * b + t); /* planted: chunk base from its own width */
#else
                const int64_t dst = i * 512 * nkb + c * 8192 + g * 64 * nb + 16 * (4 * b + t);
#endif
                memcpy(wpe + dst, we + r * (K / 2) + 16 * kb, 16);
                spe[i * 32 * nkb + c * 512 + 8 * (4 * b + t) + g] = se[r * nkb + kb];
            }
        }
    }
    return ORC_OK;
}

/* Inverse of orc_mxfp4_pack (same arguments, packed in, row-major out). */
int orc_mxfp4_unpack(int gate_up, int64_t E, int64_t I, int64_t H, const uint8_t* wp, const uint8_t* sp, uint8_t* w,
                     uint8_t* s)
{
    if (!packed_args_ok(gate_up, E, I, H) || !w || !s || !wp || !sp) return ORC_ERR_ARG;
    const int64_t R = gate_up ? 2 * I : H, K = gate_up ? H : I, nkb = K / 32;
    const int64_t items = R / 32, chunks = (nkb + 15) / 16;
    const uint8_t* src = wp;
    const uint8_t* ssrc = sp;
    for (int64_t e = 0; e < E; ++e) {
        uint8_t* we = w + e * R * (K / 2);
        uint8_t* se = s + e * R * nkb;
        for (int64_t i = 0; i < items; ++i)
            for (int64_t c = 0; c < chunks; ++c) {
                const int64_t nb = nkb - 16 * c < 16 ? nkb - 16 * c : 16;
                for (int g = 0; g < 8; ++g)
                    for (int64_t b = 0; b < nb; ++b)
                        for (int t = 0; t < 4; ++t) {
                            const int64_t r = packed_slot_row(gate_up, I, i, 4 * g + t);
                            memcpy(we + r * (K / 2) + 16 * (16 * c + b), src, 16);
                            src += 16;
                        }
                for (int64_t b = 0; b < nb; ++b)
                    for (int t = 0; t < 4; ++t)
                        for (int g = 0; g < 8; ++g) {
#if ORC_PLANT == 42
                            const int64_t r = packed_slot_row(gate_up, I, i, 4 * t + g % 4); /* planted: slot from (t, g) swapped */
#else
                            const int64_t r = packed_slot_row(gate_up, I, i, 4 * g + t);
#endif
                            se[r * nkb + 16 * c + b] = *ssrc++;
                        }
            }
    }
    return ORC_OK;
}

/* Threads the OpenMP runtime will use for a parallel region (1 without it). */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
