// Tiled grouped expert GEMM (prefill regime): many tokens per expert.
//
// Each expert segment of the permutation is an independent GEMM
//   gate/up: [M_e tokens] x [2I weight rows], K = H, A rows gathered from x
//   down:    [M_e rows of h] x [H weight rows], K = I
// with fp32 accumulation on bf16 MFMA (v_mfma_f32_16x16x32_bf16).  MXFP4
// weights (Persona Kappa post, section "Quantization-Aware Training (QAT)":
// W4A16, activations stay bf16) are decoded to bf16 while being staged into
// LDS.  The gate/up kernel computes gate and up rows of the same output
// columns in one tile and applies silu(gate)*up before writing h.
//
// Schedule: grid.y enumerates the M-tiles of all experts (expert e owns
// ceil(M_e/BM) consecutive ones; the grid is sized for the worst case
// P/BM + E and surplus blocks exit), grid.x the N-tiles.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int TL_BM = 64;       // tokens per tile
constexpr int TL_BW = 64;       // weight rows per tile (gate/up: 32 gate + 32 up)
constexpr int TL_BK = 128;      // K per stage
constexpr int TL_LD = TL_BK + 8;  // LDS row stride in bf16 (pad 16 B: conflict-free 16-B reads)
constexpr int TL_THREADS = 256;

// Stage 64 weight rows x 128 K of bf16 or MXFP4 (decoded) into Ws.
// rowof(i) gives the global row index of tile row i, or -1 for none.
template <int WFMT, typename RowOf>
__device__ __forceinline__ void stage_weights(const void* __restrict__ w, const uint8_t* __restrict__ wsc, int K,
                                              int kk, RowOf rowof, uint16_t* Ws)
{
    if constexpr (WFMT == 0) {
        // 64 rows x 16 chunks of 8 elements; 4 chunks per thread
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = threadIdx.x + TL_THREADS * q;
            const int i = c >> 4, part = c & 15;
            const long long row = rowof(i);
            const int k = kk + part * 8;
            u32x4 v = {0, 0, 0, 0};
            if (row >= 0 && k < K) v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + row * K + k);
            *reinterpret_cast<u32x4*>(Ws + i * TL_LD + part * 8) = v;
        }
    } else {
        // 64 rows x 4 blocks of 32 elements (16 bytes + 1 scale); 1 block per thread
        const int i = threadIdx.x >> 2, part = threadIdx.x & 3;
        const long long row = rowof(i);
        const int k = kk + part * 32;
        u32x4 d[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
        if (row >= 0 && k < K) {
            const u32x4 qv =
                *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w) + row * (K / 2) + k / 2);
            const float sc = e8m0_to_f32(wsc[row * (K / 32) + k / 32]);
            d[0] = fp4x8_to_bf16x8(qv.x, sc);
            d[1] = fp4x8_to_bf16x8(qv.y, sc);
            d[2] = fp4x8_to_bf16x8(qv.z, sc);
            d[3] = fp4x8_to_bf16x8(qv.w, sc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(Ws + i * TL_LD + part * 32 + q * 8) = d[q];
    }
}

// Stage 64 activation rows x 128 K (bf16) into Xs; arow(i) = row pointer or null.
template <typename ARow>
__device__ __forceinline__ void stage_acts(int K, int kk, ARow arow, uint16_t* Xs)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = threadIdx.x + TL_THREADS * q;
        const int i = c >> 4, part = c & 15;
        const uint16_t* p = arow(i);
        const int k = kk + part * 8;
        u32x4 v = {0, 0, 0, 0};
        if (p && k < K) v = *reinterpret_cast<const u32x4*>(p + k);
        *reinterpret_cast<u32x4*>(Xs + i * TL_LD + part * 8) = v;
    }
}

// One stage of MFMAs: wave w owns tokens 16w..16w+15 and all 4 weight-row
// tiles of 16.
__device__ __forceinline__ void tile_mma(const uint16_t* Ws, const uint16_t* Xs, f32x4 acc[4])
{
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < TL_BK / 32; ++q) {
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const u32x4*>(Xs + (16 * wave + r) * TL_LD + 32 * q + 8 * g));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(Ws + (16 * m + r) * TL_LD + 32 * q + 8 * g));
            acc[m] = mfma16(av, b, acc[m]);
        }
    }
}

template <int WFMT>
__global__ __launch_bounds__(TL_THREADS) void gate_up_tiled_kernel(FfnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t Ws[TL_BW * TL_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[TL_BM * TL_LD];
    __shared__ int tok[TL_BM];
    int mt;
    const int e = locate_m_tile(a.offsets, a.E, TL_BM, blockIdx.y, &mt);
    if (e < 0) return;  // uniform per block
    const int H = a.H, I = a.I;
    const int n0 = blockIdx.x * (TL_BW / 2);  // first output column (gate row)
    const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
    const int sbase = seg0 + mt * TL_BM;
    if (threadIdx.x < TL_BM) {
        const int s = sbase + threadIdx.x;
        tok[threadIdx.x] = s < seg1 ? a.sorted_pairs[s] / a.k : -1;
    }
    __syncthreads();
    auto rowof = [&](int i) -> long long {
        const int n = n0 + (i & 31);
        if (n >= I) return -1;
        return (long long)e * 2 * I + (i < 32 ? n : I + n);
    };
    auto arow = [&](int i) -> const uint16_t* { return tok[i] >= 0 ? a.x + (size_t)tok[i] * H : nullptr; };
    f32x4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    for (int kk = 0; kk < H; kk += TL_BK) {
        stage_weights<WFMT>(a.w, a.w_scale, H, kk, rowof, Ws);
        stage_acts(H, kk, arow, Xs);
        __syncthreads();
        tile_mma(Ws, Xs, acc);
        if (kk + TL_BK >= H) mfma_drain();
        __syncthreads();
    }
    // acc[0..1]: gate rows 0-15, 16-31; acc[2..3]: the matching up rows
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    const int r = lane & 15, g = lane >> 4;
    const int s = sbase + 16 * wave + r;
    if (s < seg1) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int n = n0 + 16 * m + 4 * g;
            if (n < I) {
                uint2 o;
                o.x = pack_bf16x2(silu(acc[m][0]) * acc[m + 2][0], silu(acc[m][1]) * acc[m + 2][1]);
                o.y = pack_bf16x2(silu(acc[m][2]) * acc[m + 2][2], silu(acc[m][3]) * acc[m + 2][3]);
                *reinterpret_cast<uint2*>(a.out + (size_t)s * I + n) = o;
            }
        }
    }
}

template <int WFMT>
__global__ __launch_bounds__(TL_THREADS) void down_tiled_kernel(FfnArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t Ws[TL_BW * TL_LD];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[TL_BM * TL_LD];
    int mt;
    const int e = locate_m_tile(a.offsets, a.E, TL_BM, blockIdx.y, &mt);
    if (e < 0) return;
    const int H = a.H, I = a.I;
    const int n0 = blockIdx.x * TL_BW;
    const int seg1 = a.offsets[e + 1];
    const int sbase = a.offsets[e] + mt * TL_BM;
    auto rowof = [&](int i) -> long long {
        const int n = n0 + i;
        return n < H ? (long long)e * H + n : -1;
    };
    auto arow = [&](int i) -> const uint16_t* {
        const int s = sbase + i;
        return s < seg1 ? a.a_rows + (size_t)s * I : nullptr;
    };
    f32x4 acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    for (int kk = 0; kk < I; kk += TL_BK) {
        stage_weights<WFMT>(a.w, a.w_scale, I, kk, rowof, Ws);
        stage_acts(I, kk, arow, Xs);
        __syncthreads();
        tile_mma(Ws, Xs, acc);
        if (kk + TL_BK >= I) mfma_drain();
        __syncthreads();
    }
    const int lane = lane_id(), wave = threadIdx.x / WAVE;
    const int r = lane & 15, g = lane >> 4;
    const int s = sbase + 16 * wave + r;
    if (s < seg1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int n = n0 + 16 * m + 4 * g;
            if (n < H) {
                uint2 o;
                o.x = pack_bf16x2(acc[m][0], acc[m][1]);
                o.y = pack_bf16x2(acc[m][2], acc[m][3]);
                *reinterpret_cast<uint2*>(a.out + (size_t)s * H + n) = o;
            }
        }
    }
}

static int m_tiles_bound(int P, int E) { return (P + TL_BM - 1) / TL_BM + E; }

hipError_t launch_gate_up_tiled(const FfnArgs& a, hipStream_t s)
{
    dim3 grid((a.I + TL_BW / 2 - 1) / (TL_BW / 2), m_tiles_bound(a.T * a.k, a.E));
    if (a.wfmt == 0)
        hipLaunchKernelGGL(gate_up_tiled_kernel<0>, grid, dim3(TL_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(gate_up_tiled_kernel<1>, grid, dim3(TL_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_tiled(const FfnArgs& a, hipStream_t s)
{
    dim3 grid((a.H + TL_BW - 1) / TL_BW, m_tiles_bound(a.T * a.k, a.E));
    if (a.wfmt == 0)
        hipLaunchKernelGGL(down_tiled_kernel<0>, grid, dim3(TL_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(down_tiled_kernel<1>, grid, dim3(TL_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
