// Host-side launchers of the gfx950 kernels (one .hip file per stage).
// Each returns the hipError_t of its launches; arguments are validated by the
// C-ABI layer (moe_api.hip) before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Text kept for moe_last_error() on the calling thread (C-ABI layer).
void set_last_error(const char* text);

// ------------------------------------------------------------------ route
// Exact logits (fp64 accumulation of exact bf16 products), one wave per
// (token, group of experts).  logits [T][E] fp64.
hipError_t launch_router_logits_f64(int T, int H, int E, const uint16_t* x, const uint16_t* wr, double* logits,
                                    hipStream_t s);
// Top-k by logit (ties -> lower index) + softmax over the k, one wave per token.
hipError_t launch_router_select(int T, int E, int k, const double* logits, int32_t* topk_idx, float* topk_w,
                                hipStream_t s);
// Logits + top-k + softmax: one fused matrix-core kernel when
// router_fuses_select(T, E) (logits then unused), else the two kernels above.
bool router_fuses_select(int T, int E);
hipError_t launch_router_topk(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wr, double* logits,
                              int32_t* topk_idx, float* topk_w, hipStream_t s);


// ------------------------------------------------------------------ permute
constexpr int PERMUTE_CHUNK = 1024;  // pairs ranked per workgroup pass
// Workspace for the multi-block permutation: rank [P] + hist [ceil(P/1024)][E] int32.
size_t permute_scratch_bytes(int64_t P, int E);
hipError_t launch_permute(int P, int E, const int32_t* topk_idx, int32_t* offsets, int32_t* sorted_pairs,
                          int32_t* pair_rank, void* scratch, hipStream_t s);
// True when one workgroup permutes all P pairs (then selection can be fused in).
bool permute_fits_one_block(int P);
// Top-k selection of all T tokens from logits [T][E] followed by the
// permutation, in one workgroup (requires permute_fits_one_block(T*k)).
hipError_t launch_select_permute_small(int T, int E, int k, const double* logits, int32_t* topk_idx, float* topk_w,
                                       int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_rank, hipStream_t s);

// ------------------------------------------------------------------ expert FFN
struct FfnArgs {
    int T, H, E, k, I, wfmt;   // wfmt: 0 bf16, 1 MXFP4, 2 MXFP4 in the packed order
    const uint16_t* x;          // [T][H] (gate/up input, gathered)
    const int32_t* offsets;     // [E+1]
    const int32_t* sorted_pairs;  // [P]
    const void* w;              // gate_up or down
    const uint8_t* w_scale;     // MXFP4 scales or null
    const uint16_t* a_rows;     // down: h [P][I] (sorted rows)
    // MX path: the activations split into two MXFP6 terms (launch_mx_split):
    // codes [rows][K/32][48] and scales [rows][K/32][2]; rows are tokens
    // (gate/up, gathered through sorted_pairs) or sorted pairs (down)
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    uint16_t* out;              // gate/up: h [P][I]; down: y_sorted [P][H]
    // MX gate/up only, optional: h written split for the down GEMM instead of
    // as bf16 (codes [P][I/32][48], scales [P][I/32][2]); out is then unused
    uint8_t* out_codes;
    uint8_t* out_scales;
    uint16_t* gu_out;           // tiled gate/up only, optional: g then u [P][2I] (bf16), for the backward
    // weight-gradient mode of the tiled kernel: C[e][m][n] = sum_j A_e[m][j] B_e[n][j]
    // (fp32), A_e = wg_a + wg_M * padoff[e] ([wg_M][Kpad_e]), B_e likewise with wg_N
    const uint16_t* wg_a;
    const uint16_t* wg_b;
    const int32_t* wg_padoff;   // [E+1]
    int wg_M, wg_N;
    float* wg_out;              // [E][wg_M][wg_N]
};
hipError_t launch_gate_up_skinny(const FfnArgs& a, hipStream_t s);
// The packed-MXFP4 skinny kernel addresses with 32-bit buffer offsets: true
// when a's sizes fit them.
bool skinny4_supported(const FfnArgs& a);
hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t s);
hipError_t launch_gate_up_tiled(const FfnArgs& a, hipStream_t s);
hipError_t launch_down_tiled(const FfnArgs& a, hipStream_t s);

// MX path (MXFP4 weights on the MX matrix cores).  The activations are first
// split into two MXFP6 (E2M3) terms per 32-element block, x ~ hi + lo:
// in bf16 [rows][K] -> codes [rows][K/32][48] (hi 24 B, then lo 24 B, 6 bits
// per element) + scales [rows][K/32][2] (E8M0 of hi, of lo).  K % 32 == 0.
hipError_t launch_mx_split(const uint16_t* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);
// Grouped GEMMs on v_mfma_scale_f32_32x32x64_f8f6f4 (weights E2M1, activations
// the two E2M3 terms), same outputs as launch_gate_up_tiled / launch_down_tiled;
// a.a_codes / a.a_scales hold the split activations.  Needs K % 64 == 0.
bool mx_supported(int H, int I);
hipError_t launch_gate_up_mx(const FfnArgs& a, hipStream_t s);
hipError_t launch_down_mx(const FfnArgs& a, hipStream_t s);

// ------------------------------------------------------------------ combine
hipError_t launch_combine(int T, int H, int k, const uint16_t* y_sorted, const int32_t* pair_rank,
                          const float* topk_w, uint16_t* y, hipStream_t s);

// ------------------------------------------------------------------ backward
int backward_pad_rows(int P, int E);  // rows of the per-expert padded segment buffers
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);
hipError_t launch_transpose_batched(const uint16_t* in, uint16_t* out, int nb, int R, int C, hipStream_t s);
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* padoff, uint16_t* dlT, hipStream_t s);
hipError_t launch_transpose_segments(const uint16_t* in, int C, bool gather, const int32_t* offsets,
                                     const int32_t* padoff, const int32_t* sorted_pairs, int k, int P, int E,
                                     uint16_t* out, hipStream_t s);
hipError_t launch_wgrad_tiled(const uint16_t* A, const uint16_t* B, const int32_t* padoff, int E, int M, int N,
                              float* C, hipStream_t s);
// Router weight gradient dwr [E][H] (fp32) from dlT and the token rows of x;
// part holds router_wgrad_splits(P, E) rows of H floats.
long long router_wgrad_splits(int P, int E);
hipError_t launch_router_wgrad(int H, int E, int k, int P, const int32_t* offsets, const int32_t* padoff,
                               const int32_t* sorted_pairs, const uint16_t* dlT, const uint16_t* x, float* part,
                               float* dwr, hipStream_t s);
hipError_t launch_combine_bwd(int P, int H, int k, const uint16_t* dy, const uint16_t* ys, const int32_t* sorted_pairs,
                              const float* topk_w, uint16_t* dO, float* dw, hipStream_t s);
hipError_t launch_swiglu_bwd(int P, int I, const uint16_t* da, const uint16_t* gu, uint16_t* dgu, hipStream_t s);
hipError_t launch_router_bwd(int T, int H, int k, const uint16_t* wr, const int32_t* topk_idx, const float* topk_w,
                             const float* dw, const int32_t* pair_rank, const int32_t* offsets, const int32_t* padoff,
                             const uint16_t* dxp, uint16_t* dlT, uint16_t* dx, hipStream_t s);

// ------------------------------------------------------------------ MXFP4 quantiser
// w bf16 [n_elems] (n_elems % 32 == 0) -> packed [n_elems/2] + scales
// [n_elems/32], or its decoded bf16 values.
int64_t mxfp4_quant_max_elems();
hipError_t launch_mxfp4_quantize(const uint16_t* w, int64_t n_elems, uint8_t* packed, uint8_t* scales, hipStream_t s);
hipError_t launch_mxfp4_fakequant(const uint16_t* w, int64_t n_elems, uint16_t* out, hipStream_t s);
// Row-major MXFP4 expert tensor (E experts; gate/up [2I][H] or down [H][I]) ->
// the packed MXFP4 order, bytes and scales.
hipError_t launch_mxfp4_pack(bool gate_up, int E, int I, int H, const uint8_t* w, const uint8_t* s, uint8_t* wp,
                             uint8_t* sp, hipStream_t st);

}  // namespace moe
