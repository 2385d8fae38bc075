// Weighted combine: y[t] = sum_j w[t][j] * y_sorted[pair_rank[t*k + j]].
// fp32 accumulation in slot order, one RNE rounding to bf16 at the end; each
// thread owns 8 consecutive hidden elements of one token (16-byte loads and
// stores) and issues the k row loads together.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int CB_THREADS = 64;  // one wave per (token, 512 hidden elements)

__global__ __launch_bounds__(CB_THREADS) void combine_kernel(int T, int H, int k, const uint16_t* __restrict__ ys,
                                                             const int32_t* __restrict__ pair_rank,
                                                             const float* __restrict__ topk_w,
                                                             uint16_t* __restrict__ y)
{
    const int t = blockIdx.x;
    const int c = blockIdx.y * CB_THREADS + threadIdx.x;  // 8-element chunk of the row
    if (c * 8 >= H) return;
    u32x4 v[8];
    float wk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // all k loads in flight before any arithmetic
        if (j < k) {
            v[j] = *reinterpret_cast<const u32x4*>(ys + (size_t)pair_rank[(size_t)t * k + j] * H + c * 8);
            wk[j] = topk_w[(size_t)t * k + j];
        }
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < k) {
            const uint32_t vw[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(wk[j], bf16_lo(vw[i]), acc[2 * i]);
                acc[2 * i + 1] = fmaf(wk[j], bf16_hi(vw[i]), acc[2 * i + 1]);
            }
        }
    }
    u32x4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<u32x4*>(y + (size_t)t * H + c * 8) = o;
}

hipError_t launch_combine(int T, int H, int k, const uint16_t* y_sorted, const int32_t* pair_rank,
                          const float* topk_w, uint16_t* y, hipStream_t s)
{
    dim3 grid(T, (H / 8 + CB_THREADS - 1) / CB_THREADS);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(CB_THREADS), 0, s, T, H, k, y_sorted, pair_rank, topk_w, y);
    return hipGetLastError();
}

}  // namespace moe
