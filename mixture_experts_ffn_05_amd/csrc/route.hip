// Router: logits, top-k selection and softmax over the k selected.
//
// The pages fix top-4 of 32 experts (Persona Kappa post, table "Architecture
// Summary") and 4 of 128 for the 120b model (hearth-lean-loomed-v1, section
// "Why 12-16 streams can be slow on Vulkan"), but not the selection rule.  The
// reading taken: largest logit first, an exactly equal logit goes to the lower
// expert index, weights = softmax over the k selected logits.
//
// Exactness: a bf16 x bf16 product is exact in fp64 (16 significant bits), so
// an fp64 sum of the H products differs from the exact logit by at most
// ~H * 2^-53 * sum|x*w|.  Selections therefore agree with any other fp64
// evaluation unless two logits lie within ~1e-13 relative of each other, and
// exact ties (e.g. duplicated router rows) stay exact ties.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int LOGIT_EPW = 4;  // experts per wave in the logits kernel

// One wave per (token, group of LOGIT_EPW experts).  Each lane walks its
// 8-element slices of the row (16-byte loads), accumulating exact products in
// fp64; the wave then reduces in a fixed butterfly order.
__global__ __launch_bounds__(256) void router_logits_f64_kernel(int T, int H, int E, const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ wr,
                                                                double* __restrict__ logits)
{
    const int groups = (E + LOGIT_EPW - 1) / LOGIT_EPW;
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE);
    if (wave >= T * groups) return;  // uniform per wave
    const int t = wave / groups;
    const int e0 = (wave % groups) * LOGIT_EPW;
    const int lane = lane_id();
    const uint16_t* xr = x + (size_t)t * H;
    double acc[LOGIT_EPW];
#pragma unroll
    for (int q = 0; q < LOGIT_EPW; ++q) acc[q] = 0.0;
    for (int h0 = lane * 8; h0 < H; h0 += WAVE * 8) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + h0);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < LOGIT_EPW; ++q) {
            const int e = e0 + q;
            if (e < E) {
                const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + (size_t)e * H + h0);
                const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[q] = fma((double)bf16_lo(xw[i]), (double)bf16_lo(ww[i]), acc[q]);
                    acc[q] = fma((double)bf16_hi(xw[i]), (double)bf16_hi(ww[i]), acc[q]);
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

// Does candidate (v, i) rank before (bv, bi)?  Larger logit first, then the
// lower expert index.
__device__ __forceinline__ bool ranks_before(double v, int i, double bv, int bi)
{
    return v > bv || (v == bv && i < bi);
}

// Top-k of one token's E logits (row: global or LDS) by one wave: k rounds of
// a wave-wide arg-max (each lane owns experts lane, lane+64, ...), then the
// softmax over the k selected.  Lane j writes slot j.
__device__ void wave_topk_softmax(const double* row, int E, int k, int32_t* __restrict__ idx_out,
                                  float* __restrict__ w_out)
{
    const int lane = lane_id();
    double v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + WAVE * i;
        v[i] = e < E ? row[e] : -__builtin_inf();
    }
    uint32_t taken = 0;
    double sel_v[8];
    int sel_i[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sel_v[j] = 0.0;
        sel_i[j] = 0;
        if (j < k) {
            double bv = -__builtin_inf();
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lane + WAVE * i;
                if (e < E && !(taken >> i & 1u) && ranks_before(v[i], e, bv, bi)) {
                    bv = v[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const double ov = __shfl_xor(bv, o, WAVE);
                const int oi = __shfl_xor(bi, o, WAVE);
                if (ranks_before(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            sel_v[j] = bv;
            sel_i[j] = bi;
            if ((bi & (WAVE - 1)) == lane) taken |= 1u << (bi / WAVE);
        }
    }
    double z = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) z += exp(sel_v[j] - sel_v[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < k && lane == j) {
            idx_out[j] = sel_i[j];
            w_out[j] = (float)(exp(sel_v[j] - sel_v[0]) / z);
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
    wave_topk_softmax(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

// Small batches: one workgroup per token computes all E exact logits (each
// wave takes 4 experts at a time, loads of the 4 router rows in flight
// together) into LDS, then wave 0 selects.
constexpr int RS_THREADS = 1024;
constexpr int RS_EPW = 4;

__global__ __launch_bounds__(RS_THREADS) void router_small_kernel(int H, int E, int k, const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ wr,
                                                                  int32_t* __restrict__ topk_idx,
                                                                  float* __restrict__ topk_w)
{
    __shared__ double lg[256];
    const int t = blockIdx.x;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    constexpr int NW = RS_THREADS / WAVE;
    const uint16_t* xr = x + (size_t)t * H;
    for (int e0 = wave * RS_EPW; e0 < E; e0 += NW * RS_EPW) {
        double acc[RS_EPW];
#pragma unroll
        for (int q = 0; q < RS_EPW; ++q) acc[q] = 0.0;
        for (int h0 = lane * 8; h0 < H; h0 += WAVE * 8) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + h0);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            u32x4 wv[RS_EPW];
#pragma unroll
            for (int q = 0; q < RS_EPW; ++q)
                wv[q] = e0 + q < E ? *reinterpret_cast<const u32x4*>(wr + (size_t)(e0 + q) * H + h0)
                                   : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < RS_EPW; ++q) {
                const uint32_t ww[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[q] = fma((double)bf16_lo(xw[i]), (double)bf16_lo(ww[i]), acc[q]);
                    acc[q] = fma((double)bf16_hi(xw[i]), (double)bf16_hi(ww[i]), acc[q]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < RS_EPW; ++q) {
            const double s = wave_sum(acc[q]);
            if (lane == 0 && e0 + q < E) lg[e0 + q] = s;
        }
    }
    __syncthreads();
    if (wave == 0) wave_topk_softmax(lg, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

hipError_t launch_router_small(int T, int H, int E, int k, const uint16_t* x, const uint16_t* wr, int32_t* topk_idx,
                               float* topk_w, hipStream_t s)
{
    hipLaunchKernelGGL(router_small_kernel, dim3(T), dim3(RS_THREADS), 0, s, H, E, k, x, wr, topk_idx, topk_w);
    return hipGetLastError();
}

hipError_t launch_router_logits_f64(int T, int H, int E, const uint16_t* x, const uint16_t* wr, double* logits,
                                    hipStream_t s)
{
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

}  // namespace moe
