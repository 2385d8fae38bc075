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
// an fp64 sum of the H products differs from the exact logit by at most
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

// One wave per token over precomputed logits [T][E].
__global__ __launch_bounds__(256) void router_select_kernel(int T, int E, int k, const double* __restrict__ logits,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w)
{
    const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE);
    if (t >= T) return;
    wave_topk_softmax(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
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
