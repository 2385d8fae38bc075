// Skinny-batch expert FFN: every touched expert sees only a few tokens, so the
// layer is a stream over the touched experts' weights and runs at the rate
// HBM delivers them.
//
// The pages show why this regime matters: with gpt-oss-120b at 12-16 streams
// each expert sees about one token per step, and a kernel that switches from
// mat-vec to dequantise-then-mat-mat above 8 tokens becomes ~5x slower per
// call ("hearth-lean-loomed-v1", section "Why 12-16 streams can be slow on
// Vulkan").  Here one kernel serves any token count: the tokens are the
// 16-wide N side of a bf16 MFMA (v_mfma_f32_16x16x32_bf16) whose M side is 16
// weight rows, so 1..16 tokens per expert cost the same weight traffic and
// more tokens loop over 16-token groups.  MXFP4 weights (E2M1 + E8M0 per 32
// along K; Persona Kappa post, section "Quantization-Aware Training (QAT)")
// are decoded in registers with v_cvt_scalef32_pk_bf16_fp4 and multiplied
// against bf16 activations (W4A16).
//
// Work item = (a-th touched expert, tile of 16 output rows); one wave per item.
// K is walked in super-steps of 128: lane (r, g) (r = lane % 16, g = lane / 16)
// loads 32 consecutive K elements of weight row r (64 bytes bf16 / 16 bytes
// fp4) and the same 32 elements of token r's activation row, and issues 4
// MFMAs, one per 8-element slice.  A and B use the same K order, so the dot
// product is exact in any order the MFMA reduces it.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SK_WAVES = 4;   // waves per workgroup (independent row tiles)
constexpr int SK_ROWS = 16;   // output rows per wave
constexpr int SK_KSTEP = 128; // K elements per super-step

// The lane's 32 K-values of a weight row, as 4 x 8 bf16.  `kofs` = first K
// element (multiple of 32); `valid` false -> zeros.
template <int WFMT>
__device__ __forceinline__ void load_w32(const void* __restrict__ w, const uint8_t* __restrict__ wsc, size_t row,
                                         int K, int kofs, bool valid, u32x4 out[4])
{
    if (!valid) {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = u32x4{0, 0, 0, 0};
        return;
    }
    if constexpr (WFMT == 0) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + row * K + kofs);
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __builtin_nontemporal_load(p + q);
    } else {
        const u32x4 qv = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w) + row * (K / 2) + kofs / 2));
        const float sc = e8m0_to_f32(wsc[row * (K / 32) + kofs / 32]);
        out[0] = fp4x8_to_bf16x8(qv.x, sc);
        out[1] = fp4x8_to_bf16x8(qv.y, sc);
        out[2] = fp4x8_to_bf16x8(qv.z, sc);
        out[3] = fp4x8_to_bf16x8(qv.w, sc);
    }
}

// The lane's 32 activation values (bf16 row, 64 bytes) or zeros.
__device__ __forceinline__ void load_a32(const uint16_t* __restrict__ row, int kofs, bool valid, u32x4 out[4])
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        out[q] = valid ? reinterpret_cast<const u32x4*>(row + kofs)[q] : u32x4{0, 0, 0, 0};
}

// Gate/up + SwiGLU.  grid = (ceil(I / (16*SK_WAVES)), min(E, P)).
template <int WFMT>
__global__ __launch_bounds__(SK_WAVES * WAVE) void gate_up_skinny_kernel(FfnArgs a)
{
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int n0 = (blockIdx.x * SK_WAVES + wave) * SK_ROWS;
    if (n0 >= a.I) return;  // uniform per wave
    const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
    if (e < 0) return;
    const int s0 = a.offsets[e];
    const int M = a.offsets[e + 1] - s0;
    const int r = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I;
    const size_t grow = (size_t)e * 2 * I + n0 + r;  // gate row of this lane
    const size_t urow = grow + I;                     // matching up row
    for (int j0 = 0; j0 < M; j0 += 16) {
        const int j = j0 + r;
        const bool tv = j < M;
        const uint16_t* xrow = a.x + (size_t)(tv ? a.sorted_pairs[s0 + j] / a.k : 0) * H;
        f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};

        for (int kk = 0; kk < H; kk += SK_KSTEP) {
            const int kofs = kk + 32 * g;
            const bool kv = kofs < H;
            u32x4 wg[4], wu[4], xb[4];
            load_w32<WFMT>(a.w, a.w_scale, grow, H, kofs, kv, wg);
            load_w32<WFMT>(a.w, a.w_scale, urow, H, kofs, kv, wu);
            load_a32(xrow, kofs, kv && tv, xb);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                accg = mfma16(as_bf16x8(wg[q]), as_bf16x8(xb[q]), accg);
                accu = mfma16(as_bf16x8(wu[q]), as_bf16x8(xb[q]), accu);
            }
            if (kk + SK_KSTEP >= H) mfma_drain();
        }
        if (tv) {
            // lane holds rows n0 + 4g .. +3 (gate and up alike) of token column r
            uint2 o;
            o.x = pack_bf16x2(silu(accg[0]) * accu[0], silu(accg[1]) * accu[1]);
            o.y = pack_bf16x2(silu(accg[2]) * accu[2], silu(accg[3]) * accu[3]);
            *reinterpret_cast<uint2*>(a.out + (size_t)(s0 + j) * I + n0 + 4 * g) = o;
        }
    }
}

// Down projection.  grid = (ceil(H / (16*SK_WAVES)), min(E, P)).
template <int WFMT>
__global__ __launch_bounds__(SK_WAVES * WAVE) void down_skinny_kernel(FfnArgs a)
{
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int n0 = (blockIdx.x * SK_WAVES + wave) * SK_ROWS;
    if (n0 >= a.H) return;
    const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
    if (e < 0) return;
    const int s0 = a.offsets[e];
    const int M = a.offsets[e + 1] - s0;
    const int r = lane & 15, g = lane >> 4;
    const int H = a.H, I = a.I;
    const size_t wrow = (size_t)e * H + n0 + r;
    for (int j0 = 0; j0 < M; j0 += 16) {
        const int j = j0 + r;
        const bool tv = j < M;
        const uint16_t* hrow = a.a_rows + (size_t)(s0 + (tv ? j : 0)) * I;
        f32x4 acc = {0, 0, 0, 0};

        for (int kk = 0; kk < I; kk += SK_KSTEP) {
            const int kofs = kk + 32 * g;
            const bool kv = kofs < I;
            u32x4 wv[4], hb[4];
            load_w32<WFMT>(a.w, a.w_scale, wrow, I, kofs, kv, wv);
            load_a32(hrow, kofs, kv && tv, hb);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = mfma16(as_bf16x8(wv[q]), as_bf16x8(hb[q]), acc);
            if (kk + SK_KSTEP >= I) mfma_drain();
        }
        if (tv) {
            uint2 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<uint2*>(a.out + (size_t)(s0 + j) * H + n0 + 4 * g) = o;
        }
    }
}

hipError_t launch_gate_up_skinny(const FfnArgs& a, hipStream_t s)
{
    const int P = a.T * a.k;
    dim3 grid((a.I + SK_ROWS * SK_WAVES - 1) / (SK_ROWS * SK_WAVES), P < a.E ? P : a.E);
    if (a.wfmt == 0)
        hipLaunchKernelGGL(gate_up_skinny_kernel<0>, grid, dim3(SK_WAVES * WAVE), 0, s, a);
    else
        hipLaunchKernelGGL(gate_up_skinny_kernel<1>, grid, dim3(SK_WAVES * WAVE), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t s)
{
    const int P = a.T * a.k;
    dim3 grid((a.H + SK_ROWS * SK_WAVES - 1) / (SK_ROWS * SK_WAVES), P < a.E ? P : a.E);
    if (a.wfmt == 0)
        hipLaunchKernelGGL(down_skinny_kernel<0>, grid, dim3(SK_WAVES * WAVE), 0, s, a);
    else
        hipLaunchKernelGGL(down_skinny_kernel<1>, grid, dim3(SK_WAVES * WAVE), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
