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
// more tokens take further passes over the rows.  MXFP4
// weights (E2M1 + E8M0 per 32 along K; Persona Kappa post, section
// "Quantization-Aware Training (QAT)") are decoded from LDS with
// v_cvt_scalef32_pk_bf16_fp4 and multiplied against bf16 activations (W4A16).
//
// Work item = (a-th touched expert, 32 weight rows): gate/up takes 16 gate
// rows and the 16 matching up rows, down takes 32 rows of W_down.  The rows
// are streamed in chunks of 1 KB (bf16) or 512 B (MXFP4) per row; each
// wave-wide load reads 1 KB of consecutive parts, so every access is a long
// contiguous run.  The grid is persistent: workgroup b takes items b, b+G,
// b+2G, ... (consecutive items are neighbouring rows of one expert) and walks
// the (item, token pass, chunk) sequence as one pipeline -- the next chunk,
// possibly of the next item, is fetched into registers while the current one
// is multiplied out of LDS.  The 4 waves split each chunk along K; their
// partial sums meet in LDS at the end of each item.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SK_ROWS = 32;             // weight rows per item
constexpr int SK_NG = 1;                // 16-token groups held per pass

// Per weight format: workgroup size and bytes of one row per chunk.  The
// kernel is bound by HBM latency (each workgroup keeps one chunk in flight),
// so the sizes trade chunk bytes against resident workgroups: bf16 streams
// 1 KB per row (512 elements over 4 waves, three workgroups per CU); MXFP4
// streams 512 B per row (1024 elements over 4 waves), which keeps the
// per-wave registers low enough for four workgroups per CU.
template <int WFMT>
struct SkFmt;
template <>
struct SkFmt<0> {  // bf16
    static constexpr int THREADS = 256;
    static constexpr int ROW_BYTES = 1024;
    static constexpr int KC = ROW_BYTES / 2;  // K elements per chunk
    static constexpr int MIN_WAVES = 3;       // per SIMD: 3 resident workgroups per CU
};
template <>
struct SkFmt<1> {  // MXFP4
    static constexpr int THREADS = 256;
    static constexpr int ROW_BYTES = 512;
    static constexpr int KC = ROW_BYTES * 2;
    static constexpr int MIN_WAVES = 4;       // per SIMD: 4 resident workgroups per CU
};
template <int WFMT>
struct SkGeom {
    static constexpr int THREADS = SkFmt<WFMT>::THREADS;
    static constexpr int MIN_WAVES = SkFmt<WFMT>::MIN_WAVES;
    static constexpr int WAVES = THREADS / WAVE;
    static constexpr int ROW_BYTES = SkFmt<WFMT>::ROW_BYTES;
    static constexpr int LDROW = ROW_BYTES + 16;                 // LDS row stride (16-B pad: conflict-free reads)
    static constexpr int KC = SkFmt<WFMT>::KC;
    static constexpr int STEPS = KC / WAVES / 32;                // MFMA K-steps per wave per chunk
    static constexpr int PARTS = ROW_BYTES / 16;                 // 16-B parts per row per chunk
    static constexpr int LOADS = SK_ROWS * PARTS / THREADS;      // 16-B loads per thread per chunk
    static constexpr int SCROW = KC / 32;                        // MXFP4 scale bytes per row per chunk
    static constexpr int SCB = SK_ROWS * SCROW / THREADS;        // scale bytes per thread per chunk
    static_assert(SK_ROWS * PARTS % THREADS == 0 && STEPS * WAVES * 32 == KC, "chunk geometry");
};

template <int WFMT>
struct SkShared {
    uint8_t w[SK_ROWS * SkGeom<WFMT>::LDROW];                   // weight chunk
    uint8_t sc[SK_ROWS * SkGeom<WFMT>::SCROW];                  // MXFP4 scales of the chunk
    f32x4 red[SkGeom<WFMT>::WAVES * 2 * SK_NG * WAVE];          // per-wave partial sums of an item
};

// Position in a workgroup's pipeline: which item, token pass and K chunk.
struct SkCursor {
    int item;  // -1: past the end
    int e, n0, s0, M;
    int j0, kc;
};

template <bool GATE_UP>
__device__ __forceinline__ size_t sk_row(int e, int i, int n0, int N)
{
    if constexpr (GATE_UP)  // N = I: rows 0-15 gate n0.., rows 16-31 up n0..
        return (size_t)e * 2 * N + (i < 16 ? n0 + i : N + n0 + (i - 16));
    else  // N = H
        return (size_t)e * N + n0 + i;
}

// Number of experts with a non-empty segment (one wave).
__device__ __forceinline__ int count_active(const int32_t* __restrict__ offsets, int E)
{
    int n = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane_id();
        n += __popcll(ballot(e < E && offsets[e + 1] > offsets[e]));
    }
    return n;
}

template <bool GATE_UP>
__device__ __forceinline__ SkCursor sk_item(const FfnArgs& a, int item, int n_items, int tiles)
{
    SkCursor c;
    c.item = item < n_items ? item : -1;
    c.j0 = 0;
    c.kc = 0;
    c.e = c.n0 = c.s0 = c.M = 0;
    if (c.item >= 0) {
        c.e = nth_active_expert(a.offsets, a.E, item / tiles);
        c.n0 = (item % tiles) * (GATE_UP ? 16 : 32);
        c.s0 = a.offsets[c.e];
        c.M = a.offsets[c.e + 1] - c.s0;
    }
    return c;
}

// Next (chunk | token pass | item) after c.
template <int WFMT, bool GATE_UP>
__device__ __forceinline__ SkCursor sk_next(const FfnArgs& a, const SkCursor& c, int K, int n_items, int tiles)
{
    SkCursor n = c;
    n.kc += SkFmt<WFMT>::KC;
    if (n.kc < K) return n;
    n.kc = 0;
    n.j0 += 16 * SK_NG;
    if (n.j0 < n.M) return n;
    return sk_item<GATE_UP>(a, c.item + gridDim.x, n_items, tiles);
}

// Fetch chunk c.kc of item c's 32 rows into registers: load j of thread t
// takes 16-B part f = j*THREADS + t, i.e. row f / PARTS, part f % PARTS, so a
// wave-wide load reads 1 KB of consecutive parts.  Parts past K read as zero.
template <int WFMT, bool GATE_UP>
__device__ __forceinline__ void sk_fetch(const FfnArgs& a, const SkCursor& c, int N, int K,
                                         u32x4 (&v)[SkGeom<WFMT>::LOADS], uint32_t (&s)[SkGeom<WFMT>::SCB])
{
    using G = SkGeom<WFMT>;
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) {
        const int f = j * G::THREADS + threadIdx.x;
        const int part = f % G::PARTS;
        const size_t row = sk_row<GATE_UP>(c.e, f / G::PARTS, c.n0, N);
        if constexpr (WFMT == 0) {
            const int k = c.kc + part * 8;
            v[j] = k < K ? __builtin_nontemporal_load(
                               reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.w) + row * K + k))
                         : u32x4{0, 0, 0, 0};
        } else {
            const int k = c.kc + part * 32;
            v[j] = k < K ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                               static_cast<const uint8_t*>(a.w) + row * (K / 2) + k / 2))
                         : u32x4{0, 0, 0, 0};
        }
    }
    if constexpr (WFMT == 1) {  // scales: SCB consecutive bytes of one row per thread
        constexpr int PER_ROW = G::SCROW / G::SCB;
        const int i = threadIdx.x / PER_ROW, b0 = (threadIdx.x % PER_ROW) * G::SCB;
        const uint8_t* p = a.w_scale + sk_row<GATE_UP>(c.e, i, c.n0, N) * (K / 32) + c.kc / 32 + b0;
        const int left = K / 32 - (c.kc / 32 + b0);
#pragma unroll
        for (int b = 0; b < G::SCB; ++b) s[b] = b < left ? p[b] : 0u;
    }
}

template <int WFMT>
__device__ __forceinline__ void sk_store(SkShared<WFMT>& sh, const u32x4 (&v)[SkGeom<WFMT>::LOADS],
                                         const uint32_t (&s)[SkGeom<WFMT>::SCB])
{
    using G = SkGeom<WFMT>;
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) {
        const int f = j * G::THREADS + threadIdx.x;
        *reinterpret_cast<u32x4*>(sh.w + (f / G::PARTS) * G::LDROW + (f % G::PARTS) * 16) = v[j];
    }
    if constexpr (WFMT == 1) {
        constexpr int PER_ROW = G::SCROW / G::SCB;
        const int i = threadIdx.x / PER_ROW, b0 = (threadIdx.x % PER_ROW) * G::SCB;
        static_assert(G::SCB % 2 == 0, "scales stored as 16-bit pairs");
#pragma unroll
        for (int b = 0; b < G::SCB; b += 2)
            *reinterpret_cast<uint16_t*>(sh.sc + i * G::SCROW + b0 + b) = (uint16_t)(s[b] | (s[b + 1] << 8));
    }
}

// A operand: 8 weights of tile row r (tile t = rows 16t..16t+15) at chunk-local
// K offset kl (multiple of 8), as bf16x8.
template <int WFMT>
__device__ __forceinline__ bf16x8 sk_a(const SkShared<WFMT>& sh, int t, int r, int kl)
{
    using G = SkGeom<WFMT>;
    const int row = 16 * t + r;
    if constexpr (WFMT == 0) {
        return as_bf16x8(*reinterpret_cast<const u32x4*>(sh.w + row * G::LDROW + kl * 2));
    } else {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(sh.w + row * G::LDROW + kl / 2);
        return as_bf16x8(fp4x8_to_bf16x8(q, e8m0_to_f32(sh.sc[row * G::SCROW + kl / 32])));
    }
}

// Activation row of token j0 + 16q + (lane % 16) of the item's expert, or null.
template <bool GATE_UP>
__device__ __forceinline__ const uint16_t* sk_arow(const FfnArgs& a, const SkCursor& c, int q)
{
    const int j = c.j0 + 16 * q + (lane_id() & 15);
    if (j >= c.M) return nullptr;
    if constexpr (GATE_UP)
        return a.x + (size_t)(a.sorted_pairs[c.s0 + j] / a.k) * a.H;
    else
        return a.a_rows + (size_t)(c.s0 + j) * a.I;
}

// Write the item's outputs for one token pass from the summed partials.
template <int WFMT, bool GATE_UP>
__device__ __forceinline__ void sk_epilogue(const FfnArgs& a, const SkShared<WFMT>& sh, const SkCursor& c)
{
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    auto sum = [&](int t, int q) {
        f32x4 s = sh.red[(t * SK_NG + q) * WAVE + lane];
#pragma unroll
        for (int w = 1; w < SkGeom<WFMT>::WAVES; ++w) s += sh.red[((w * 2 + t) * SK_NG + q) * WAVE + lane];
        return s;
    };
    if constexpr (GATE_UP) {
        if (wave < SK_NG) {
            const int j = c.j0 + 16 * wave + r;
            if (j < c.M) {
                const f32x4 gv = sum(0, wave), uv = sum(1, wave);
                uint2 o;
                o.x = pack_bf16x2(silu(gv[0]) * uv[0], silu(gv[1]) * uv[1]);
                o.y = pack_bf16x2(silu(gv[2]) * uv[2], silu(gv[3]) * uv[3]);
                *reinterpret_cast<uint2*>(a.out + (size_t)(c.s0 + j) * a.I + c.n0 + 4 * g) = o;
            }
        }
    } else {
        if (wave < 2 * SK_NG) {
            const int t = wave & 1, q = wave >> 1;
            const int j = c.j0 + 16 * q + r;
            if (j < c.M) {
                const f32x4 v = sum(t, q);
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(a.out + (size_t)(c.s0 + j) * a.H + c.n0 + 16 * t + 4 * g) = o;
            }
        }
    }
}

// Persistent skinny kernel.  gate/up: N = I output columns, K = H;
// down: N = H output rows, K = I.
template <int WFMT, bool GATE_UP>
__global__ __launch_bounds__(SkGeom<WFMT>::THREADS, SkGeom<WFMT>::MIN_WAVES) void skinny_kernel(FfnArgs a)
{
    using F = SkGeom<WFMT>;
    __shared__ __attribute__((aligned(16))) SkShared<WFMT> sh;
    const int N = GATE_UP ? a.I : a.H;
    const int K = GATE_UP ? a.H : a.I;
    const int tiles = GATE_UP ? N / 16 : N / 32;
    const int n_items = count_active(a.offsets, a.E) * tiles;
    SkCursor cur = sk_item<GATE_UP>(a, blockIdx.x, n_items, tiles);
    if (cur.item < 0) return;  // uniform per block

    const int wave = threadIdx.x / WAVE, lane = lane_id();
    const int r = lane & 15, g = lane >> 4;
    const int kw = wave * F::STEPS * 32;  // this wave's K offset inside a chunk

    u32x4 pre[F::LOADS];
    uint32_t spre[F::SCB];
    sk_fetch<WFMT, GATE_UP>(a, cur, N, K, pre, spre);
    sk_store<WFMT>(sh, pre, spre);
    __syncthreads();

    f32x4 acc[2][SK_NG];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < SK_NG; ++q) acc[t][q] = f32x4{0, 0, 0, 0};
    const uint16_t* arow[SK_NG];
#pragma unroll
    for (int q = 0; q < SK_NG; ++q) arow[q] = sk_arow<GATE_UP>(a, cur, q);

    while (true) {
        const SkCursor nxt = sk_next<WFMT, GATE_UP>(a, cur, K, n_items, tiles);
        const bool last_chunk = nxt.item != cur.item || nxt.j0 != cur.j0;
        if (nxt.item >= 0) sk_fetch<WFMT, GATE_UP>(a, nxt, N, K, pre, spre);
        if (cur.kc + kw < K) {  // waves whose K range lies past the end skip the tail chunk
            // all of this chunk's activations (L2-resident, one latency), then the MFMAs
            u32x4 b[F::STEPS][SK_NG];
#pragma unroll
            for (int s = 0; s < F::STEPS; ++s) {
                const int k = cur.kc + kw + 32 * s + 8 * g;
#pragma unroll
                for (int q = 0; q < SK_NG; ++q)
                    b[s][q] = (arow[q] && k < K) ? *reinterpret_cast<const u32x4*>(arow[q] + k) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int s = 0; s < F::STEPS; ++s) {
                const int kl = kw + 32 * s + 8 * g;
                const bf16x8 a0 = sk_a<WFMT>(sh, 0, r, kl);
                const bf16x8 a1 = sk_a<WFMT>(sh, 1, r, kl);
#pragma unroll
                for (int q = 0; q < SK_NG; ++q) {
                    acc[0][q] = mfma16(a0, as_bf16x8(b[s][q]), acc[0][q]);
                    acc[1][q] = mfma16(a1, as_bf16x8(b[s][q]), acc[1][q]);
                }
                // MXFP4: keep at most two steps of decoded operands live (the
                // scheduler would otherwise hoist all of them and spill)
                if constexpr (WFMT == 1)
                    if (s % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (last_chunk) {
            mfma_drain();
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int q = 0; q < SK_NG; ++q) {
                    sh.red[((wave * 2 + t) * SK_NG + q) * WAVE + lane] = acc[t][q];
                    acc[t][q] = f32x4{0, 0, 0, 0};
                }
        }
        __syncthreads();  // all waves are done with sh.w (and have published sh.red)
        if (last_chunk) sk_epilogue<WFMT, GATE_UP>(a, sh, cur);
        if (nxt.item < 0) break;
        sk_store<WFMT>(sh, pre, spre);
        if (last_chunk) {
#pragma unroll
            for (int q = 0; q < SK_NG; ++q) arow[q] = sk_arow<GATE_UP>(a, nxt, q);
        }
        __syncthreads();  // next chunk visible; sh.red free again
        cur = nxt;
    }
}

// Resident workgroups of `kernel` on the whole device (the persistent grid:
// items are assigned round-robin by block index, so every block must be
// resident from the start).
static int resident_blocks(const void* kernel, int threads)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    return cus * per_cu;
}

template <int WFMT, bool GATE_UP>
static hipError_t launch_skinny(const FfnArgs& a, hipStream_t s)
{
    constexpr int threads = SkGeom<WFMT>::THREADS;
    static const int cap = resident_blocks(reinterpret_cast<const void*>(&skinny_kernel<WFMT, GATE_UP>), threads);
    const int P = a.T * a.k;
    const int tiles = GATE_UP ? a.I / 16 : a.H / 32;
    const long long bound = (long long)(P < a.E ? P : a.E) * tiles;
    const int grid = (int)(bound < cap ? bound : cap);
    hipLaunchKernelGGL((skinny_kernel<WFMT, GATE_UP>), dim3(grid), dim3(threads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up_skinny(const FfnArgs& a, hipStream_t s)
{
    return a.wfmt == 0 ? launch_skinny<0, true>(a, s) : launch_skinny<1, true>(a, s);
}

hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t s)
{
    return a.wfmt == 0 ? launch_skinny<0, false>(a, s) : launch_skinny<1, false>(a, s);
}

}  // namespace moe
