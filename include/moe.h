/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts FFN layer library.
 *
 * The layer is the gpt-oss expert block: each token is routed to the top k of
 * E experts by a linear router, each selected expert applies a SwiGLU FFN, and
 * the k expert outputs are summed with the routing weights.  The pages fix the
 * shapes and number formats:
 *   - hidden 2880, top-4 of 32 experts, SwiGLU experts: "Persona Kappa:
 *     training a 20B LLM on desktop GPUs" (Level1Techs forum), table
 *     "Architecture Summary";
 *   - 4 of 128 experts for the 120b model, ~1 token per expert at 12-16
 *     streams: "hearth-lean-loomed-v1" model card, section "Why 12-16 streams
 *     can be slow on Vulkan";
 *   - expert weights natively MXFP4, activations kept in bf16 (W4A16), and
 *     2880 not a multiple of 128: Persona Kappa post, section
 *     "Quantization-Aware Training (QAT)"; "gpt-oss-20b" model page, section
 *     "Architecture";
 *   - bf16 forward with fp32 accumulation: Persona Kappa post, section
 *     "Techniques That Made It Fit".
 * The pages give no formulas; the library computes (T tokens, H hidden, E
 * experts, k per token, I expert width, P = T*k pairs):
 *   l[t][e]   = sum_h x[t][h] * W_router[e][h]
 *   slots     = the k experts with the largest l[t][.], largest first; an
 *               exactly equal logit goes to the lower expert index
 *   w[t][j]   = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k slots
 *   pair p    = t*k + j, routed to expert topk_idx[t][j]
 *   g, u      = x[t] . W_gate_up[e][0..I-1][:],  x[t] . W_gate_up[e][I..2I-1][:]
 *   h         = silu(g) * u,   silu(z) = z / (1 + exp(-z))
 *   o         = W_down[e] . h
 *   y[t]      = sum_j w[t][j] * o_{t,j}        (j in slot order)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers (HIP global memory) unless stated otherwise;
 * `dims` and `weights` structs are HOST memory read during the call.
 * All matrices are row-major with the last index contiguous.  bf16 buffers
 * hold raw bfloat16 bit patterns.
 *
 *   x              bf16  [T][H]
 *   w_router       bf16  [E][H]
 *   gate_up  bf16  bf16  [E][2I][H]     rows 0..I-1 gate, rows I..2I-1 up
 *   down     bf16  bf16  [E][H][I]
 *   gate_up  MXFP4 u8    [E][2I][H/2]   + gate_up_scale u8 [E][2I][H/32]
 *   down     MXFP4 u8    [E][H][I/2]    + down_scale    u8 [E][H][I/32]
 *            (OCP MX: E2M1 element 2b in the low nibble of byte b, element
 *             2b+1 in the high nibble; one E8M0 scale 2^(S-127) per 32
 *             consecutive elements along the input dimension)
 *   gate_up, down  MXFP4 in the packed order (MOE_WFMT_MXFP4_PACKED): the same
 *            bytes and scales, same array sizes, reordered by moe_mxfp4_pack
 *            (the order is defined there)
 *   topk_idx       int32 [T][k]   slots in routing order
 *   topk_w         fp32  [T][k]
 *   expert_offsets int32 [E+1]    exclusive prefix sum of pairs per expert
 *   sorted_pairs   int32 [P]      pair ids p, expert-major, ascending p within
 *                                 an expert (a stable sort by expert)
 *   pair_rank      int32 [P]      inverse: pair_rank[sorted_pairs[s]] = s
 *   h              bf16  [P][I]   SwiGLU output, row s = sorted position
 *   y_sorted       bf16  [P][H]   unweighted expert outputs, row s = sorted position
 *   y              bf16  [T][H]
 *
 * Expert weights may also live in pinned host memory, passed as the device
 * address of the mapping (hipHostGetDevicePointer): in the skinny regime the
 * kernels then read only the touched experts' rows over the host link, once
 * per layer (the pinned-host-bank streaming that the pages' serving engines
 * use for models larger than the GPU's memory; "gpt-oss-20b" model page,
 * section "llama-swap.yaml entry").
 *
 * Alignment: bf16 matrices, weight bytes and the workspace must be 16-byte
 * aligned; int32/fp32 arrays 4-byte aligned; row-major scale arrays need no
 * alignment, packed-order scale arrays 8 bytes.
 * Supported sizes: 1 <= E <= 256, 1 <= k <= min(E, 8), H and I multiples of
 * 32, T >= 0 with T*k < 2^31.  T = 0 returns MOE_OK and launches nothing.
 *
 * Ownership: the caller owns every buffer, including the workspace (size from
 * moe_workspace_size).  The library allocates nothing, frees nothing and keeps
 * no state between calls.  Outputs must not alias inputs.
 *
 * Asynchrony: each call validates its arguments on the host, then only
 * enqueues kernels on `stream` (a hipStream_t passed as void*; NULL = the
 * default stream) and returns; there is no host synchronisation and no
 * device-to-host copy.  Buffers must stay valid until the stream has run the
 * work.  Results are deterministic: the same inputs give bitwise-identical
 * outputs (no split-K, no floating-point atomics).
 *
 * Errors: every call returns an int (MOE_OK or an error code below).  All
 * validation happens before the first launch: on error nothing is launched
 * and no output is touched.  A launch failure returns MOE_ERR_HIP; the HIP
 * error text is kept per thread for moe_last_error().  No C++ exception
 * crosses this interface.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, negative size, k < 1 or k > E, T*k overflow */
    MOE_ERR_UNSUPPORTED = 2, /* E > 256, k > 8, H or I not a multiple of 32, unknown wfmt/path */
    MOE_ERR_MISALIGNED = 3,  /* a pointer breaks the alignment rules above */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_size() */
    MOE_ERR_HIP = 5          /* a HIP launch failed; see moe_last_error() */
};

/* Expert weight formats.  MXFP4_PACKED holds MXFP4 weights in the packed
 * order of moe_mxfp4_pack: every path accepts it, and the skinny (decode)
 * regime streams it as long contiguous runs.  Its skinny kernel addresses
 * with 32-bit offsets: it needs I*H < 2^31, T*H < 2^30 and T*k*I < 2^30.
 * Outside those sizes MOE_PATH_SKINNY returns MOE_ERR_UNSUPPORTED and
 * MOE_PATH_AUTO takes the tiled path. */
enum { MOE_WFMT_BF16 = 0, MOE_WFMT_MXFP4 = 1, MOE_WFMT_MXFP4_PACKED = 2 };

/* Expert-FFN schedule.  AUTO picks SKINNY when tokens per expert are few
 * (weight streaming at HBM rate) and TILED otherwise (LDS-tiled grouped GEMM).
 * For MXFP4 weights the tiled regime has two kernels:
 *   TILED_DEQUANT  E2M1 x E8M0 decoded exactly to bf16 while staged into LDS,
 *                  bf16 MFMA (W4A16 as the pages describe it: "Persona Kappa:
 *                  training a 20B LLM on desktop GPUs", section
 *                  "Quantization-Aware Training (QAT)");
 *   TILED_MX       the weights fed as stored to the MX matrix cores
 *                  (v_mfma_scale_f32_32x32x64_f8f6f4), the bf16 activations
 *                  split per 32-value block into two MXFP6 (E2M3) terms,
 *                  x ~ hi + lo (see moe_mx_split); needs H and I multiples
 *                  of 64, else MOE_ERR_UNSUPPORTED.  Its rounding differs
 *                  from the bf16 path's (hi + lo keeps about as much of each
 *                  activation as bf16 does; both stay within the layer's
 *                  1e-2 * max|y| tolerance), so the two give different bits.
 * TILED (and AUTO in the tiled regime) takes TILED_MX wherever it applies,
 * else TILED_DEQUANT: on the 20b MXFP4 prefill the MX kernel is the faster of
 * the two.  moe_gate_up and moe_down then need the workspace (the split
 * activations live there); moe_grouped_ffn and moe_forward keep h only in its
 * split form, made by the gate/up kernel, with the same bits as the stage
 * entry points give.  For bf16 weights all tiled paths are the bf16 kernel
 * except TILED_MX, which returns MOE_ERR_UNSUPPORTED.  Every path computes
 * the same function; forcing one is for testing and tuning. */
enum {
    MOE_PATH_AUTO = 0,
    MOE_PATH_SKINNY = 1,
    MOE_PATH_TILED = 2,
    MOE_PATH_TILED_DEQUANT = 3,
    MOE_PATH_TILED_MX = 4
};

typedef struct moe_dims {
    int32_t T, H, E, k, I;
    int32_t wfmt; /* MOE_WFMT_* : format of gate_up and down */
    int32_t path; /* MOE_PATH_* */
} moe_dims;

typedef struct moe_expert_weights {
    const void* gate_up;          /* see layouts above */
    const uint8_t* gate_up_scale; /* MXFP4 only, else NULL */
    const void* down;
    const uint8_t* down_scale;    /* MXFP4 only, else NULL */
} moe_expert_weights;

/* Workspace bytes needed by every entry point below for these dims (the
 * largest, moe_forward's, covers all).  Host-only; launches nothing. */
int moe_workspace_size(const moe_dims* dims, size_t* bytes);

/* Router (logits, top-k selection, softmax over the k selected).
 * Reads x, w_router; writes topk_idx [T][k], topk_w [T][k].
 * Each logit is an fp64 sum of the H bf16 x bf16 products (each exact in
 * fp64); the summation order differs between kernels, so a logit may differ
 * from the exact sum by up to about H * 2^-53 * sum_h |x[h] * w[h]|.  Indices
 * therefore match any double-precision reference unless two of a token's
 * logits lie that close together; exactly equal logits (duplicated router
 * rows) stay exactly equal and go to the lower index.  A NaN logit ranks
 * below every number (as -infinity), so the k indices of a token are always
 * distinct and in [0, E): a token whose logits are all NaN (a NaN in its x
 * row) gets experts 0..k-1 and NaN weights; other tokens are unaffected. */
int moe_route(const moe_dims* dims, const void* x, const void* w_router, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream);

/* Permutation of the P pairs into expert-contiguous segments (stable counting
 * sort by expert).  Reads topk_idx; writes expert_offsets [E+1],
 * sorted_pairs [P], pair_rank [P].  topk_idx values outside [0, E) are
 * undefined behaviour (moe_route never produces them, whatever its input). */
int moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_pairs,
                int32_t* pair_rank, void* workspace, size_t workspace_bytes, void* stream);

/* Gate/up projection with the fused SwiGLU epilogue, per expert segment:
 * h[s] = silu(x[t] . Wg^T) * (x[t] . Wu^T) for sorted position s of pair
 * p = sorted_pairs[s], t = p / k.  Writes h [P][I] (bf16, fp32 accumulate). */
int moe_gate_up(const moe_dims* dims, const void* x, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                const moe_expert_weights* weights, void* h, void* workspace, size_t workspace_bytes, void* stream);

/* Down projection per expert segment: y_sorted[s] = W_down[e] . h[s] for
 * every s in expert e's segment.  Writes y_sorted [P][H] (bf16, unweighted). */
int moe_down(const moe_dims* dims, const void* h, const int32_t* expert_offsets, const moe_expert_weights* weights,
             void* y_sorted, void* workspace, size_t workspace_bytes, void* stream);

/* moe_gate_up followed by moe_down, with h kept in the workspace. */
int moe_grouped_ffn(const moe_dims* dims, const void* x, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                    const moe_expert_weights* weights, void* y_sorted, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Weighted combine: y[t] = sum_j topk_w[t][j] * y_sorted[pair_rank[t*k+j]],
 * summed in fp32 in slot order, rounded to bf16 (nearest-even). */
int moe_combine(const moe_dims* dims, const void* y_sorted, const int32_t* pair_rank, const float* topk_w, void* y,
                void* stream);

/* The whole layer: route, permute, gate/up + SwiGLU, down, combine.
 * topk_idx_out / topk_w_out may be NULL (then they live in the workspace);
 * when given they receive the routing. */
int moe_forward(const moe_dims* dims, const void* x, const void* w_router, const moe_expert_weights* weights, void* y,
                int32_t* topk_idx_out, float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing: the intermediates live in a
 * library-owned device array of MOE_NOALLOC_SCRATCH_BYTES (32 MiB), one per
 * GPU, held from library load until the process ends.  Arguments, results and
 * errors as moe_forward; in addition MOE_ERR_WORKSPACE when
 * moe_workspace_size(dims) exceeds MOE_NOALLOC_SCRATCH_BYTES (for the
 * 2880-wide layers with k = 4: up to about 700 tokens).  Nothing in the array
 * needs clearing between calls (every call writes what it later reads).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller.  The first call on a device looks up the array's address
 * (hipGetSymbolAddress) with that device current; a failure there returns
 * MOE_ERR_HIP. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_forward_noalloc(const moe_dims* dims, const void* x, const void* w_router, const moe_expert_weights* weights,
                        void* y, int32_t* topk_idx_out, float* topk_w_out, void* stream);

/* Backward of moe_forward (the training variant: full-parameter fine-tuning,
 * "kappa-20b-131k" model card; bf16 with fp32 accumulation and activations
 * recomputed during backprop, "Persona Kappa: training a 20B LLM on desktop
 * GPUs", section "Techniques That Made It Fit"), for
 * bf16 weights (dims->wfmt = MOE_WFMT_BF16, else MOE_ERR_UNSUPPORTED).
 * Given the upstream gradient dy bf16 [T][H] of the layer output y, it
 * recomputes the forward (routing, permutation, gate/up, down) and writes the
 * gradients of L = sum_t dy[t] . y[t]:
 *   dx         bf16 [T][H]      w.r.t. x: through the experts and the router
 *   dw_router  fp32 [E][H]      w.r.t. w_router
 *   dgate_up   fp32 [E][2I][H]  w.r.t. weights->gate_up (gate rows, then up)
 *   ddown      fp32 [E][H][I]   w.r.t. weights->down
 * Per slot j of token t with expert e: dw_j = dy . o_j, do_j = w_j dy,
 * da = Wd^T do_j, dg = da * u * silu'(g), du = da * silu(g),
 * dx += Wg^T dg + Wu^T du, dWd[e] += do_j a^T, dWgu[e] += [dg; du] x^T; per
 * token through the softmax over the k selected logits,
 * dl_j = w_j (dw_j - sum_i w_i dw_i), dx += sum_j dl_j Wr[e_j],
 * dWr[e_j] += dl_j x.  The top-k selection itself is piecewise constant and
 * passes no gradient.  The expert products run on bf16 MFMA with fp32
 * accumulation, dWr on fp32 vector FMAs in a fixed order (sums over 64-row
 * splits of each expert's sorted rows, then the splits in order);
 * intermediates (w dy, g and u, [dg; du], per-pair dx, dl) are stored in bf16.
 * An expert that receives no token gets zero weight gradients; T = 0 writes
 * zeros to the three weight gradients and touches nothing else.
 * Workspace: moe_backward_workspace_size() bytes (it includes the forward's
 * workspace).  Alignment as above; the fp32 outputs need 4 bytes.  Outputs
 * must not overlap inputs or each other. */
int moe_backward_workspace_size(const moe_dims* dims, size_t* bytes);
int moe_backward(const moe_dims* dims, const void* x, const void* w_router, const moe_expert_weights* weights,
                 const void* dy, void* dx, float* dw_router, float* dgate_up, float* ddown, void* workspace,
                 size_t workspace_bytes, void* stream);

/* MXFP4 quantisation of bf16 weights: the step that produces MXFP4 expert
 * weights from bf16 ones ("Persona Kappa: training a 20B LLM on desktop
 * GPUs", section "Quantization-Aware Training (QAT)": after training through
 * fake-quantised expert weights, the weights are exported quantised).  The
 * pages give no rounding rule; this is OCP Microscaling v1.0's.  Per block of
 * 32 consecutive elements of a row of w bf16 [rows][cols], with amax the
 * largest |v| of the block:
 *   S = clamp(floor(log2 amax) - 2 + 127, 0, 254)  stored in scales
 *       u8 [rows][cols/32]; an all-zero block stores S = 0;
 *   each element v / 2^(S-127) rounded to the nearest E2M1 value, an exact
 *   midpoint to the even code, stored in packed u8 [rows][cols/2] (element
 *   2b in the low nibble of byte b); a zero code never carries the sign bit.
 * This is the layout the layer's MXFP4 weights use, so a [E][N][K] bf16
 * tensor quantises with rows = E*N, cols = K.  Inf/NaN inputs give undefined
 * codes.  Errors: rows or cols < 0 -> MOE_ERR_INVALID_ARG; cols % 32 != 0 or
 * rows*cols too large for one launch (over 2^41 elements) ->
 * MOE_ERR_UNSUPPORTED;
 * w or packed not 16-byte aligned -> MOE_ERR_MISALIGNED; a null pointer ->
 * MOE_ERR_INVALID_ARG.  rows*cols = 0 returns MOE_OK and launches nothing.
 * Outputs must not overlap w.  Asynchronous on `stream` like every call. */
int moe_mxfp4_quantize(int64_t rows, int32_t cols, const void* w, uint8_t* packed, uint8_t* scales, void* stream);

/* Fake quantisation, the forward of training through quantisation (same
 * section): out bf16 [rows][cols] = the decoded values of
 * moe_mxfp4_quantize(w), E2M1(code) * 2^(S-127).  Every such value is exactly
 * a bf16 value, so out is exact.  Same arguments rules as moe_mxfp4_quantize;
 * out must be 16-byte aligned and must not overlap w. */
int moe_mxfp4_fakequant(int64_t rows, int32_t cols, const void* w, void* out, void* stream);

/* Packed MXFP4 order: reorders one MXFP4 expert tensor (bytes and scales) for
 * weight streaming in the decode regime.  This is the library's own storage
 * order, not the pages': they fix the MXFP4 format ("Persona Kappa: training
 * a 20B LLM on desktop GPUs", section "Quantization-Aware Training (QAT)"),
 * and the packed order changes no byte or scale value, it only moves them.
 * It is a one-time step at weight load; the layer then runs with
 * dims->wfmt = MOE_WFMT_MXFP4_PACKED.
 *
 * which = MOE_PACK_GATE_UP: w [E][2I][H/2], scales [E][2I][H/32] (K = H);
 * which = MOE_PACK_DOWN:    w [E][H][I/2],  scales [E][H][I/32]  (K = I).
 * Per expert a piece is the 16 bytes of one row over K-block kb (elements
 * 32kb..32kb+31) and it carries that block's scale.  Rows form items of 32
 * slots: a gate/up item i holds gate rows 16i..16i+15 (slots 0-15) and the
 * matching up rows I+16i..I+16i+15 (slots 16-31); a down item i holds rows
 * 32i..32i+31.  With slot q = 4g + t (g < 8, t < 4), kb = 16c + b (b < 16),
 * nkb = K/32 and nb(c) = min(16, nkb - 16c), the piece of (item i, slot q,
 * kb) goes to byte i*512*nkb + c*8192 + g*64*nb(c) + 16*(4b + t) of the
 * expert's packed bytes and its scale to byte i*32*nkb + c*512 + 8*(4b + t)
 * + g of the expert's packed scales; experts keep the row-major strides.
 * Outputs w_packed [same size as w], scales_packed [same size as scales].
 * Uses dims->E, H, I (validated as for the layer; T, k, path are checked
 * but unused).  Errors: dims invalid -> as moe_forward; which not one of
 * MOE_PACK_* or a null pointer -> MOE_ERR_INVALID_ARG; w or w_packed not
 * 16-byte aligned or scales_packed not 8-byte aligned -> MOE_ERR_MISALIGNED;
 * an output overlapping an input or the other output -> MOE_ERR_INVALID_ARG.
 * Asynchronous on `stream` like every call. */
enum { MOE_PACK_GATE_UP = 0, MOE_PACK_DOWN = 1 };
int moe_mxfp4_pack(const moe_dims* dims, int32_t which, const uint8_t* w, const uint8_t* scales, uint8_t* w_packed,
                   uint8_t* scales_packed, void* stream);

/* The activation split of the MX path (MOE_PATH_TILED_MX): bf16 x [rows][cols]
 * (cols % 32 == 0) as two MXFP6 terms per block of 32 consecutive elements of
 * a row.  With amax the block's largest |x| and
 *   S  = clamp(floor(log2 amax) - 2 + 127, 1, 254)   (OCP Microscaling v1.0
 *        shared exponent for E2M3, whose largest exponent is 2),
 *   hi = each x / 2^(S-127) rounded to the nearest E2M3 value (ties to the
 *        even code, saturating at +-7.5), times 2^(S-127),
 *   lo = x - hi (exact), encoded the same way with its own S2 from its amax,
 * it writes codes u8 [rows][cols/32][48]: the block's 32 hi codes (6 bits
 * each, element j at bits 6j..6j+5 of the 24 bytes, little-endian), then its
 * 32 lo codes; and scales u8 [rows][cols/32][2]: S, then S2.  E2M3 codes:
 * sign bit 5, exponent bits 4:3 (bias 1), mantissa bits 2:0.  The layer's MX
 * path makes these itself in its workspace; this entry point is for callers
 * and tests.  Errors: rows < 0 or a null pointer -> MOE_ERR_INVALID_ARG;
 * cols % 32 != 0 or cols <= 0 -> MOE_ERR_UNSUPPORTED; x or codes not 16-byte
 * aligned, scales not 2-byte aligned -> MOE_ERR_MISALIGNED.  rows = 0 returns
 * MOE_OK.  Inputs are finite; a NaN or Inf element gives undefined codes for
 * its block.  Asynchronous on `stream` like every call. */
int moe_mx_split(int64_t rows, int32_t cols, const void* x, uint8_t* codes, uint8_t* scales, void* stream);

/* Static text for an error code. */
const char* moe_strerror(int code);

/* Text of the last MOE_ERR_HIP raised on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
