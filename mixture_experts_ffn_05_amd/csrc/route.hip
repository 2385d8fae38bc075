// Router: logits, top-k selection and softmax over the k selected.
//
// The pages fix top-4 of 32 experts (Persona Kappa post, table "Architecture
// Summary") and 4 of 128 for the 120b model (hearth-lean-loomed-v1, section
// "Why 12-16 streams can be slow on Vulkan"), but not the selection rule; the
// rule implemented by wave_topk_softmax (moe_device.h) is: largest logit
// first, an exactly equal logit goes to the lower expert index, weights =
// softmax over the k selected logits.
//
// Exactness: a bf16 x bf16 product is exact in fp64 (16 significant bits), so
// an fp64 sum of the H products (in any order: both logit kernels below use
// fp64 accumulation) differs from the exact logit by at most
// ~H * 2^-53 * sum|x*w|.  Selections therefore agree with any other fp64
// evaluation unless two logits lie within ~1e-13 relative of each other, and
// exact ties (e.g. duplicated router rows) stay exact ties.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int LOGIT_EPW = 2;  // experts per wave in the logits kernel
constexpr int LOGIT_HU = 6;   // 16-byte slices per lane per pass (3072 hidden elements)

// One wave per (token, pair of experts).  Each lane issues all of its 16-byte
// loads of the x row and the two router rows for up to 3072 hidden elements
// at once, accumulates the exact products in fp64, and the wave reduces in a
// fixed butterfly order.  Router rows are spread over many waves (and CUs),
// so no single CU streams the whole router matrix.
__global__ __launch_bounds__(256) void router_logits_f64_kernel(int T, int H, int E, const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ wr,
                                                                double* __restrict__ logits)
{
    const int groups = (E + LOGIT_EPW - 1) / LOGIT_EPW;
    const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / WAVE;
    if (wave >= (long long)T * groups) return;  // uniform per wave
    const int t = (int)(wave / groups);
    const int e0 = (int)(wave % groups) * LOGIT_EPW;
    const int lane = lane_id();
    const uint16_t* xr = x + (size_t)t * H;
    double acc[LOGIT_EPW];
#pragma unroll
    for (int q = 0; q < LOGIT_EPW; ++q) acc[q] = 0.0;
    for (int hb = 0; hb < H; hb += WAVE * 8 * LOGIT_HU) {
        u32x4 xv[LOGIT_HU], wv[LOGIT_EPW][LOGIT_HU];
#pragma unroll
        for (int i = 0; i < LOGIT_HU; ++i) {
            const int h = hb + WAVE * 8 * i + lane * 8;
            const bool ok = h < H;
            xv[i] = ok ? *reinterpret_cast<const u32x4*>(xr + h) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < LOGIT_EPW; ++q)
                wv[q][i] = (ok && e0 + q < E) ? *reinterpret_cast<const u32x4*>(wr + (size_t)(e0 + q) * H + h)
                                              : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LOGIT_HU; ++i) {
            const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
            for (int q = 0; q < LOGIT_EPW; ++q) {
                const uint32_t ww[4] = {wv[q][i].x, wv[q][i].y, wv[q][i].z, wv[q][i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[q] = fma((double)bf16_lo(xw[j]), (double)bf16_lo(ww[j]), acc[q]);
                    acc[q] = fma((double)bf16_hi(xw[j]), (double)bf16_hi(ww[j]), acc[q]);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < LOGIT_EPW; ++q) {
        const double s = wave_sum(acc[q]);
        if (lane == 0 && e0 + q < E) logits[(size_t)t * E + e0 + q] = s;
    }
}

// Many tokens: the logits as an fp64 matrix product on the matrix cores
// (v_mfma_f64_16x16x4_f64; fp64 rate as the vector units, with operands fed
// from registers).  A workgroup owns 16 tokens x 32 or 64 experts; its 4 waves split
// H in blocks of 32 (wave w takes blocks w, w+4, ...) and their partial sums
// meet in LDS.  MFMA operand layout: lane l supplies A[l%16][l/16] (token
// l%16) and B[l/16][l%16] (expert l%16); D[4e + l/16][l%16] is element e of
// lane l.  Inside a block, lane group g = l/16 loads 8 consecutive hidden
// elements h0+8g..h0+8g+7 of its token row and of its experts' router rows,
// and MFMA step s takes element s of them as its k-index g, so the 8 steps
// cover the block's 32 products once, each exact in fp64.  A workgroup takes
// two 16-expert tiles when E <= 32, else four.
constexpr int RL_WAVES = 4;
constexpr int RL_D = 3;  // 32-element blocks of H in flight per wave

typedef __attribute__((ext_vector_type(4))) double f64x4;

__device__ __forceinline__ void bf16x8_to_f64(u32x4 v, double (&d)[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d[2 * i] = (double)bf16_lo(w[i]);
        d[2 * i + 1] = (double)bf16_hi(w[i]);
    }
}

// With SELECT (all E experts in this workgroup's tiles), wave 0 also takes
// the top k of each of its 16 tokens and their softmax weights, and the
// logits are not written.
template <int RL_ET, bool SELECT>  // RL_ET: 16-expert tiles per workgroup
__global__ __launch_bounds__(RL_WAVES * WAVE) void router_logits_mfma_kernel(int T, int H, int E, int k,
                                                                              const uint16_t* __restrict__ x,
                                                                              const uint16_t* __restrict__ wr,
                                                                              double* __restrict__ logits,
                                                                              int32_t* __restrict__ topk_idx,
                                                                              float* __restrict__ topk_w)
{
    __shared__ f64x4 red[RL_WAVES - 1][RL_ET][WAVE];
    const int t0 = blockIdx.x * 16, eg = blockIdx.y * 16 * RL_ET;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    // rows past T or E re-read the last valid row; their results are not stored
    const uint16_t* xr = x + (size_t)min(t0 + r, T - 1) * H + 8 * g;
    const uint16_t* wrow[RL_ET];
#pragma unroll
    for (int j = 0; j < RL_ET; ++j) wrow[j] = wr + (size_t)min(eg + 16 * j + r, E - 1) * H + 8 * g;
    f64x4 acc[RL_ET];
#pragma unroll
    for (int j = 0; j < RL_ET; ++j) acc[j] = f64x4{0, 0, 0, 0};

    // Wave w takes blocks w, w + RL_WAVES, ...; RL_D of them are in flight in
    // a ring of registers indexed by compile-time slots.  The loads are not
    // conditional (a block index past the end reads the last block again, in
    // bounds and unused), so no register is merged or copied between loop
    // trips and the wait before a block's MFMAs covers only its own loads.
    // A slot's operands are converted before its next block's loads are
    // issued into it.
    const int nb = H / 32;  // H is a multiple of 32
    u32x4 xv[RL_D], wv[RL_D][RL_ET];
    auto load = [&](int sl, int b) {
        const int bc = min(b, nb - 1);
        xv[sl] = *reinterpret_cast<const u32x4*>(xr + 32 * bc);
#pragma unroll
        for (int j = 0; j < RL_ET; ++j) wv[sl][j] = *reinterpret_cast<const u32x4*>(wrow[j] + 32 * bc);
    };
#pragma unroll
    for (int sl = 0; sl < RL_D; ++sl) load(sl, wave + RL_WAVES * sl);
    int b0 = wave;
    for (; b0 + RL_WAVES * (RL_D - 1) < nb; b0 += RL_WAVES * RL_D) {  // all RL_D slots hold blocks
#pragma unroll
        for (int sl = 0; sl < RL_D; ++sl) {
            double xd[8], wd[RL_ET][8];
            bf16x8_to_f64(xv[sl], xd);
#pragma unroll
            for (int j = 0; j < RL_ET; ++j) bf16x8_to_f64(wv[sl][j], wd[j]);
            load(sl, b0 + RL_WAVES * (sl + RL_D));
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int j = 0; j < RL_ET; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[s], wd[j][s], acc[j], 0, 0, 0);
            // keep the next slot's conversions (and so its wait) after these MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int sl = 0; sl < RL_D - 1; ++sl) {  // the last blocks, already loaded
        if (b0 + RL_WAVES * sl >= nb) break;  // uniform
        double xd[8], wd[RL_ET][8];
        bf16x8_to_f64(xv[sl], xd);
#pragma unroll
        for (int j = 0; j < RL_ET; ++j) bf16x8_to_f64(wv[sl][j], wd[j]);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int j = 0; j < RL_ET; ++j)
                acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[s], wd[j][s], acc[j], 0, 0, 0);
    }
    mfma_drain();  // accumulators are read right after the loop
    if (wave > 0) {
#pragma unroll
        for (int j = 0; j < RL_ET; ++j) red[wave - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (wave != 0) return;
    f64x4 v[RL_ET];
#pragma unroll
    for (int j = 0; j < RL_ET; ++j) {
        v[j] = acc[j];
#pragma unroll
        for (int w = 0; w < RL_WAVES - 1; ++w) v[j] += red[w][j][lane];
    }
    if constexpr (!SELECT) {
#pragma unroll
        for (int j = 0; j < RL_ET; ++j) {
            const int e = eg + 16 * j + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 4 * i + g;
                if (t < T && e < E) logits[(size_t)t * E + e] = v[j][i];
            }
        }
    } else {
        // Token t0 + 4i + g is held by the 16 lanes of group g (expert 16j + r
        // in element i of tile j): k rounds of arg-max within the group
        // (largest logit, an exactly equal one to the lower index; NaN ranks
        // as -infinity), then the softmax over the k, in the same arithmetic
        // as router_select_kernel.
#pragma unroll
        for (int j = 0; j < RL_ET; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[j][i] = rank_key(v[j][i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * i + g;
            uint32_t taken = 0;
            double sel_v[8];
            int sel_i[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                sel_v[q] = 0.0;
                sel_i[q] = 0;
                if (q < k) {
                    double bv = -__builtin_inf();
                    int bi = 0x7FFFFFFF;
#pragma unroll
                    for (int j = 0; j < RL_ET; ++j) {
                        const int e = 16 * j + r;
                        if (e < E && !(taken >> j & 1u) && ranks_before(v[j][i], e, bv, bi)) {
                            bv = v[j][i];
                            bi = e;
                        }
                    }
#pragma unroll
                    for (int o = 8; o > 0; o >>= 1) {
                        const double ov = __shfl_xor(bv, o, WAVE);
                        const int oi = __shfl_xor(bi, o, WAVE);
                        if (ranks_before(ov, oi, bv, bi)) {
                            bv = ov;
                            bi = oi;
                        }
                    }
                    sel_v[q] = bv;
                    sel_i[q] = bi;
                    if ((bi & 15) == r) taken |= 1u << (bi >> 4);
                }
            }
            double z = 0.0;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q < k) z += exp(sel_v[q] - sel_v[0]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (q < k && r == q && t < T) {
                    topk_idx[(size_t)t * k + q] = sel_i[q];
                    topk_w[(size_t)t * k + q] = (float)(exp(sel_v[q] - sel_v[0]) / z);
                }
            }
        }
    }
}

// One wave per token over precomputed logits [T][E].
__global__ __launch_bounds__(256) void router_select_kernel(int T, int E, int k, const double* __restrict__ logits,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w)
{
    const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE);
    if (t >= T) return;
    if (E <= WAVE)
        wave_topk_softmax_rank(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
    else
        wave_topk_softmax(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

// Token count from which the matrix-core kernel replaces the per-token waves.
constexpr int RL_MFMA_MIN_T = 1024;

hipError_t launch_router_logits_f64(int T, int H, int E, const uint16_t* x, const uint16_t* wr, double* logits,
                                    hipStream_t s)
{
    if (T >= RL_MFMA_MIN_T) {
        const dim3 block(RL_WAVES * WAVE);
        if (E <= 32)
            hipLaunchKernelGGL((router_logits_mfma_kernel<2, false>), dim3((T + 15) / 16, 1), block, 0, s, T, H, E, 0, x,
                               wr, logits, nullptr, nullptr);
        else
            hipLaunchKernelGGL((router_logits_mfma_kernel<4, false>), dim3((T + 15) / 16, (E + 63) / 64), block, 0, s,
                               T, H, E, 0, x, wr, logits, nullptr, nullptr);
        return hipGetLastError();
    }
    const int groups = (E + LOGIT_EPW - 1) / LOGIT_EPW;
    const long long waves = (long long)T * groups;
    const int blocks = (int)((waves + 3) / 4);
    hipLaunchKernelGGL(router_logits_f64_kernel, dim3(blocks), dim3(256), 0, s, T, H, E, x, wr, logits);
    return hipGetLastError();
}

hipError_t launch_router_select(int T, int E, int k, const double* logits, int32_t* topk_idx, float* topk_w,
                                hipStream_t s)
{
    const int blocks = (T + 3) / 4;
    hipLaunchKernelGGL(router_select_kernel, dim3(blocks), dim3(256), 0, s, T, E, k, logits, topk_idx, topk_w);
    return hipGetLastError();
}

bool router_fuses_select(int T, int E) { return T >= RL_MFMA_MIN_T && E <= 64; }

hipError_t launch_router_topk(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wr, double* logits,
                              int32_t* topk_idx, float* topk_w, hipStream_t s)
{
    if (router_fuses_select(T, E)) {
        const dim3 grid((T + 15) / 16), block(RL_WAVES * WAVE);
        if (E <= 32)
            hipLaunchKernelGGL((router_logits_mfma_kernel<2, true>), grid, block, 0, s, T, H, E, k, x, wr, nullptr,
                               topk_idx, topk_w);
        else
            hipLaunchKernelGGL((router_logits_mfma_kernel<4, true>), grid, block, 0, s, T, H, E, k, x, wr, nullptr,
                               topk_idx, topk_w);
        return hipGetLastError();
    }
    hipError_t err = launch_router_logits_f64(T, H, E, x, wr, logits, s);
    if (err != hipSuccess) return err;
    return launch_router_select(T, E, k, logits, topk_idx, topk_w, s);
}


}  // namespace moe
