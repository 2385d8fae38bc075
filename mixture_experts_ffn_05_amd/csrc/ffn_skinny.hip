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
// weight rows, so 1..16 tokens per expert cost the same weight traffic, up to
// 32 tokens are held at once, and more tokens take further passes.  MXFP4
// weights (E2M1 + E8M0 per 32 along K; Persona Kappa post, section
// "Quantization-Aware Training (QAT)") are decoded from LDS with
// v_cvt_scalef32_pk_bf16_fp4 and multiplied against bf16 activations (W4A16).
//
// Work item = (a-th touched expert, 32 weight rows): gate/up takes 16 gate
// rows and the 16 matching up rows, down takes 32 rows of W_down.  The rows
// are streamed in chunks of 1 KB per row (512 bf16 or 2048 fp4 elements):
// each wave-wide load reads 1 KB of one row, so every access is a long
// contiguous run.  Chunk c+1 is fetched into registers while chunk c is
// multiplied out of LDS; the 4 waves split each chunk along K and their
// partial sums meet in LDS at the end.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SK_THREADS = 256;
constexpr int SK_WAVES = SK_THREADS / WAVE;
constexpr int SK_ROWS = 32;             // weight rows per block
constexpr int SK_ROW_BYTES = 1024;      // bytes of one row per chunk
constexpr int SK_LDROW = SK_ROW_BYTES + 16;  // LDS row stride (16-B pad: conflict-free operand reads)
constexpr int SK_NG = 2;                // 16-token groups held per pass
constexpr int SK_LOADS = SK_ROWS * SK_ROW_BYTES / 16 / SK_THREADS;  // 16-B loads per thread per chunk (8)

template <int WFMT>
struct SkFmt;
template <>
struct SkFmt<0> {  // bf16
    static constexpr int KC = SK_ROW_BYTES / 2;          // K elements per chunk
    static constexpr int STEPS = KC / SK_WAVES / 32;    // MFMA K-steps per wave per chunk (4)
};
template <>
struct SkFmt<1> {  // MXFP4
    static constexpr int KC = SK_ROW_BYTES * 2;
    static constexpr int STEPS = KC / SK_WAVES / 32;    // 16
};

struct SkShared {
    uint8_t w[SK_ROWS * SK_LDROW];  // weight chunk; reused for the cross-wave reduction
    uint8_t sc[SK_ROWS * 64];       // MXFP4 scales of the chunk (KC/32 per row)
};

// Global row index of block row i (0..31).
template <bool GATE_UP>
__device__ __forceinline__ size_t sk_row(int e, int i, int n0, int N)
{
    if constexpr (GATE_UP)  // N = I: rows 0-15 gate n0.., rows 16-31 up n0..
        return (size_t)e * 2 * N + (i < 16 ? n0 + i : N + n0 + (i - 16));
    else  // N = H
        return (size_t)e * N + n0 + i;
}

// Fetch chunk kc of the block's 32 rows into registers (8 x 16 B per thread;
// wave w, load j reads 1 KB of row w + 4j).  Parts past K read as zero.
template <int WFMT, bool GATE_UP>
__device__ __forceinline__ void sk_fetch(const void* __restrict__ w, int e, int n0, int N, int K, int kc,
                                         u32x4 (&v)[SK_LOADS])
{
    const int part = lane_id(), w0 = threadIdx.x / WAVE;
#pragma unroll
    for (int j = 0; j < SK_LOADS; ++j) {
        const size_t row = sk_row<GATE_UP>(e, w0 + SK_WAVES * j, n0, N);
        if constexpr (WFMT == 0) {
            const int k = kc + part * 8;
            v[j] = k < K ? __builtin_nontemporal_load(
                               reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(w) + row * K + k))
                         : u32x4{0, 0, 0, 0};
        } else {
            const int k = kc + part * 32;
            v[j] = k < K ? __builtin_nontemporal_load(
                               reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w) + row * (K / 2) + k / 2))
                         : u32x4{0, 0, 0, 0};
        }
    }
}

// MXFP4 scales of chunk kc: thread t loads 8 bytes of row t/8.
template <bool GATE_UP>
__device__ __forceinline__ void sk_fetch_scales(const uint8_t* __restrict__ wsc, int e, int n0, int N, int K, int kc,
                                                uint32_t (&s)[8])
{
    const int i = threadIdx.x >> 3, b0 = (threadIdx.x & 7) * 8;
    const uint8_t* p = wsc + sk_row<GATE_UP>(e, i, n0, N) * (K / 32) + kc / 32 + b0;
    const int left = K / 32 - (kc / 32 + b0);
#pragma unroll
    for (int b = 0; b < 8; ++b) s[b] = b < left ? p[b] : 0u;
}

__device__ __forceinline__ void sk_store(SkShared& sh, const u32x4 (&v)[SK_LOADS])
{
    const int part = lane_id(), w0 = threadIdx.x / WAVE;
#pragma unroll
    for (int j = 0; j < SK_LOADS; ++j)
        *reinterpret_cast<u32x4*>(sh.w + (w0 + SK_WAVES * j) * SK_LDROW + part * 16) = v[j];
}

__device__ __forceinline__ void sk_store_scales(SkShared& sh, const uint32_t (&s)[8])
{
    const int i = threadIdx.x >> 3, b0 = (threadIdx.x & 7) * 8;
    uint2 packed;
    packed.x = s[0] | (s[1] << 8) | (s[2] << 16) | (s[3] << 24);
    packed.y = s[4] | (s[5] << 8) | (s[6] << 16) | (s[7] << 24);
    *reinterpret_cast<uint2*>(sh.sc + i * 64 + b0) = packed;
}

// A operand: 8 weights of tile row r (tile t = rows 16t..16t+15) at chunk-local
// K offset kl (multiple of 8), as bf16x8.
template <int WFMT>
__device__ __forceinline__ bf16x8 sk_a(const SkShared& sh, int t, int r, int kl)
{
    const int row = 16 * t + r;
    if constexpr (WFMT == 0) {
        return as_bf16x8(*reinterpret_cast<const u32x4*>(sh.w + row * SK_LDROW + kl * 2));
    } else {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(sh.w + row * SK_LDROW + kl / 2);
        return as_bf16x8(fp4x8_to_bf16x8(q, e8m0_to_f32(sh.sc[row * 64 + kl / 32])));
    }
}

// One pass over the block's rows for up to SK_NG*16 tokens (row pointers
// arow, null = no token).  Leaves per-wave partial sums in acc[tile][group].
template <int WFMT, bool GATE_UP>
__device__ __forceinline__ void sk_pass(const FfnArgs& a, SkShared& sh, int e, int n0, int N, int K,
                                        const uint16_t* const (&arow)[SK_NG], f32x4 (&acc)[2][SK_NG])
{
    using F = SkFmt<WFMT>;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    const int kw = wave * F::STEPS * 32;  // this wave's K offset inside a chunk
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < SK_NG; ++q) acc[t][q] = f32x4{0, 0, 0, 0};

    u32x4 pre[SK_LOADS];
    uint32_t spre[8];
    sk_fetch<WFMT, GATE_UP>(a.w, e, n0, N, K, 0, pre);
    if constexpr (WFMT == 1) sk_fetch_scales<GATE_UP>(a.w_scale, e, n0, N, K, 0, spre);
    sk_store(sh, pre);
    if constexpr (WFMT == 1) sk_store_scales(sh, spre);
    __syncthreads();
    for (int kc = 0; kc < K; kc += F::KC) {
        const bool more = kc + F::KC < K;
        // activations of this chunk first (L2-resident), then the next weight chunk (HBM)
        constexpr int BATCH = 4;
#pragma unroll
        for (int s0 = 0; s0 < F::STEPS; s0 += BATCH) {
            u32x4 b[BATCH][SK_NG];
#pragma unroll
            for (int s = 0; s < BATCH; ++s) {
                const int k = kc + kw + 32 * (s0 + s) + 8 * g;
#pragma unroll
                for (int q = 0; q < SK_NG; ++q)
                    b[s][q] = (arow[q] && k < K) ? *reinterpret_cast<const u32x4*>(arow[q] + k) : u32x4{0, 0, 0, 0};
            }
            if (s0 == 0 && more) {
                sk_fetch<WFMT, GATE_UP>(a.w, e, n0, N, K, kc + F::KC, pre);
                if constexpr (WFMT == 1) sk_fetch_scales<GATE_UP>(a.w_scale, e, n0, N, K, kc + F::KC, spre);
            }
#pragma unroll
            for (int s = 0; s < BATCH; ++s) {
                const int kl = kw + 32 * (s0 + s) + 8 * g;
                const bf16x8 a0 = sk_a<WFMT>(sh, 0, r, kl);
                const bf16x8 a1 = sk_a<WFMT>(sh, 1, r, kl);
#pragma unroll
                for (int q = 0; q < SK_NG; ++q) {
                    acc[0][q] = mfma16(a0, as_bf16x8(b[s][q]), acc[0][q]);
                    acc[1][q] = mfma16(a1, as_bf16x8(b[s][q]), acc[1][q]);
                }
            }
        }
        if (!more) mfma_drain();
        __syncthreads();
        if (more) {
            sk_store(sh, pre);
            if constexpr (WFMT == 1) sk_store_scales(sh, spre);
            __syncthreads();
        }
    }
}

// Publish this wave's partial sums to LDS (sh.w must be free: the pass ended
// with a barrier); all threads call.
__device__ __forceinline__ void sk_reduce_publish(SkShared& sh, const f32x4 (&acc)[2][SK_NG])
{
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    f32x4* red = reinterpret_cast<f32x4*>(sh.w);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < SK_NG; ++q) red[((wave * 2 + t) * SK_NG + q) * WAVE + lane] = acc[t][q];
    __syncthreads();
}

// Sum of the 4 waves' partials of (tile t, group q) for this lane, in wave order.
__device__ __forceinline__ f32x4 sk_reduce_get(const SkShared& sh, int t, int q)
{
    const int lane = lane_id();
    const f32x4* red = reinterpret_cast<const f32x4*>(sh.w);
    f32x4 s = red[(t * SK_NG + q) * WAVE + lane];
#pragma unroll
    for (int w = 1; w < SK_WAVES; ++w) s += red[((w * 2 + t) * SK_NG + q) * WAVE + lane];
    return s;
}

// gate/up + SwiGLU.  grid = (I / 16, min(E, P)).
template <int WFMT>
__global__ __launch_bounds__(SK_THREADS) void gate_up_skinny_kernel(FfnArgs a)
{
    __shared__ __attribute__((aligned(16))) SkShared sh;
    const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
    if (e < 0) return;  // uniform per block
    const int n0 = blockIdx.x * 16;
    const int s0 = a.offsets[e], M = a.offsets[e + 1] - s0;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    for (int j0 = 0; j0 < M; j0 += 16 * SK_NG) {
        const uint16_t* arow[SK_NG];
#pragma unroll
        for (int q = 0; q < SK_NG; ++q) {
            const int j = j0 + 16 * q + r;
            arow[q] = j < M ? a.x + (size_t)(a.sorted_pairs[s0 + j] / a.k) * a.H : nullptr;
        }
        f32x4 acc[2][SK_NG];
        sk_pass<WFMT, true>(a, sh, e, n0, a.I, a.H, arow, acc);
        sk_reduce_publish(sh, acc);
        if (wave < SK_NG) {
            const int j = j0 + 16 * wave + r;
            if (j < M) {
                const f32x4 gv = sk_reduce_get(sh, 0, wave), uv = sk_reduce_get(sh, 1, wave);
                uint2 o;
                o.x = pack_bf16x2(silu(gv[0]) * uv[0], silu(gv[1]) * uv[1]);
                o.y = pack_bf16x2(silu(gv[2]) * uv[2], silu(gv[3]) * uv[3]);
                *reinterpret_cast<uint2*>(a.out + (size_t)(s0 + j) * a.I + n0 + 4 * g) = o;
            }
        }
        __syncthreads();  // sh.w is reused by the next pass
    }
}

// Down projection.  grid = (H / 32, min(E, P)).
template <int WFMT>
__global__ __launch_bounds__(SK_THREADS) void down_skinny_kernel(FfnArgs a)
{
    __shared__ __attribute__((aligned(16))) SkShared sh;
    const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
    if (e < 0) return;
    const int n0 = blockIdx.x * 32;
    const int s0 = a.offsets[e], M = a.offsets[e + 1] - s0;
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    for (int j0 = 0; j0 < M; j0 += 16 * SK_NG) {
        const uint16_t* arow[SK_NG];
#pragma unroll
        for (int q = 0; q < SK_NG; ++q) {
            const int j = j0 + 16 * q + r;
            arow[q] = j < M ? a.a_rows + (size_t)(s0 + j) * a.I : nullptr;
        }
        f32x4 acc[2][SK_NG];
        sk_pass<WFMT, false>(a, sh, e, n0, a.H, a.I, arow, acc);
        sk_reduce_publish(sh, acc);
        if (wave < 2 * SK_NG) {
            const int t = wave & 1, q = wave >> 1;
            const int j = j0 + 16 * q + r;
            if (j < M) {
                const f32x4 v = sk_reduce_get(sh, t, q);
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(a.out + (size_t)(s0 + j) * a.H + n0 + 16 * t + 4 * g) = o;
            }
        }
        __syncthreads();
    }
}

hipError_t launch_gate_up_skinny(const FfnArgs& a, hipStream_t s)
{
    const int P = a.T * a.k;
    dim3 grid(a.I / 16, P < a.E ? P : a.E);
    if (a.wfmt == 0)
        hipLaunchKernelGGL(gate_up_skinny_kernel<0>, grid, dim3(SK_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(gate_up_skinny_kernel<1>, grid, dim3(SK_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t s)
{
    const int P = a.T * a.k;
    dim3 grid(a.H / 32, P < a.E ? P : a.E);
    if (a.wfmt == 0)
        hipLaunchKernelGGL(down_skinny_kernel<0>, grid, dim3(SK_THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(down_skinny_kernel<1>, grid, dim3(SK_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
