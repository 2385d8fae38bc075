// Skinny-batch expert FFN: every touched expert sees only a few tokens, so the
// layer is a stream over the touched experts' weights and runs at the rate
// HBM delivers them.
//
// The pages show why this regime matters: routing top-4 of 128 experts for
// 12 to 16 concurrent streams leaves roughly one token per expert per decode
// step, and the engine they measure loses about 5x per expert call when it
// leaves its mat-vec kernel for a dequantise-then-mat-mat one above 8 tokens
// ("hearth-lean-loomed-v1", section "Why 12-16 streams can be slow on
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


// ---------------------------------------------------------------------------
// MXFP4 skinny kernel on v_mfma_f32_4x4x4_16b_bf16.  That instruction runs 16
// independent 4x4x4 products per wave: lane (block b, t) supplies row t of
// the block's A and column t of its B, each with 4 consecutive K values, and
// receives column t of the block's 4x4 result.  Here every block owns its own
// K range, so a block multiplies 4 weight rows by 4 tokens over K-block b
// (32 K) of each 512-K chunk, and only the real tokens' activations are
// loaded: lane (b, t) loads token t's 32 bf16 at that K-block (64 B), where a
// 16x16 MFMA would move 16 token columns whatever the count.  A wave item is
// 32 weight rows (8 groups of 4; gate/up: 16 gate rows then the 16 matching
// up rows) and 4 or 8 tokens per pass (TG groups of 4; a pass with at most 4
// tokens multiplies only the first group).  Per chunk lane
// (b, t) loads, from HBM straight into registers, the 16 bytes of E2M1 codes
// of row 4g+t at its K-block for each group g with the 8 scale bytes, and
// token 4*tg+t's activations; the E2M1 codes are decoded once and used by the
// TG token groups.  No LDS and no barrier: waves are independent.  After the
// last chunk of a pass the 16 blocks' partial sums are added across lanes.
//
// It reads weights in the packed MXFP4 order (documented with moe_mxfp4_pack),
// which makes each group's 16-byte pieces 1 KB of consecutive bytes per wave
// load and puts a lane's 8 scale bytes in one 8-byte word.  (Row-major MXFP4
// weights are served by skinny_kernel above: read this way, each wave load
// would cover 4 rows x 256 B and the scales would take 8 byte loads per chunk,
// which streams slower.)
constexpr int S4_RG = 8;                 // 4-row groups per item (32 rows)
constexpr int S4_KB = 16;                // K-blocks per chunk, one per MFMA block
constexpr int S4_KC = S4_KB * 32;        // K per chunk
constexpr int S4_THREADS = 256;
constexpr int S4_WPB = S4_THREADS / WAVE;
constexpr uint32_t S4_OOB = 0x80000000u; // buffer offset past every range: loads return zero
typedef __attribute__((ext_vector_type(4))) short s16x4;

struct S4Cursor {
    int item;  // -1: past the end
    int e, it, s0, M, j0, kc;  // expert, item inside the expert, segment, token pass, K chunk
};

template <int TG>
struct S4Buf {
    u32x4 w[S4_RG];    // E2M1 codes of row 4g+t at this lane's K-block
    uint32_t s[2];     // the 8 scale bytes, one per group
    u32x4 x[TG][4];    // token 4*tg+t: 32 bf16 at this lane's K-block
};

__device__ __forceinline__ f32x4 mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c)
{
    const s16x4 a = __builtin_bit_cast(s16x4, uint2{a0, a1});
    const s16x4 b = __builtin_bit_cast(s16x4, uint2{b0, b1});
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// The layer's expert segments, read once per wave: bit l of mask[j] says
// expert 64j + l has tokens; this lane holds offsets[64j + lane] and
// offsets[64j + lane + 1].  Items are decoded from it without memory access,
// so a wave moving to its next item never waits on its loads in flight.
struct S4Experts {
    uint64_t mask[4];
    int lo[4], hi[4];
    int active;  // experts with tokens
};

__device__ __forceinline__ S4Experts s4_experts(const FfnArgs& a)
{
    S4Experts x;
    x.active = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // E <= 256
        const int e = 64 * j + lane_id();
        x.lo[j] = e < a.E ? a.offsets[e] : 0;
        x.hi[j] = e < a.E ? a.offsets[e + 1] : 0;
        x.mask[j] = ballot(x.hi[j] > x.lo[j]);
        x.active += __popcll(x.mask[j]);
    }
    return x;
}

__device__ __forceinline__ S4Cursor s4_item(const S4Experts& x, int item, int n_items, int tiles)
{
    S4Cursor c;
    c.item = item < n_items ? item : -1;
    c.j0 = c.kc = 0;
    c.e = c.it = c.s0 = c.M = 0;
    if (c.item >= 0) {
        int r = item / tiles;  // rank of the expert among those with tokens
        c.it = item % tiles;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cnt = __popcll(x.mask[j]);
            if (r >= 0 && r < cnt) {
                const uint32_t lo = (uint32_t)x.mask[j], hi = (uint32_t)(x.mask[j] >> 32);
                const int before = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
                const uint64_t hit = ballot(((x.mask[j] >> lane_id()) & 1) && before == r);
                const int l = (int)__builtin_ctzll(hit);
                c.e = 64 * j + l;
                c.s0 = __builtin_amdgcn_readlane(x.lo[j], l);
                c.M = __builtin_amdgcn_readlane(x.hi[j], l) - c.s0;
            }
            r -= cnt;
        }
    }
    return c;
}

template <int TG>
__device__ __forceinline__ S4Cursor s4_next(const S4Experts& x, const S4Cursor& c, int K, int n_items, int tiles,
                                            int nw)
{
    S4Cursor n = c;
    if (c.item < 0) return n;
    n.kc += S4_KC;
    if (n.kc < K) return n;
    n.kc = 0;
    n.j0 += 4 * TG;
    if (n.j0 < n.M) return n;
    return s4_item(x, c.item + nw, n_items, tiles);
}

// Pair indices of this lane's tokens in cursor c's pass (gate/up only), as
// buffer loads so that they are in flight one step ahead of their use.
template <int TG>
__device__ __forceinline__ void s4_pairs(const FfnArgs& a, const S4Cursor& c, uint32_t (&p)[TG])
{
    const int t = lane_id() & 3;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.sorted_pairs), (short)0, a.T * a.k * 4, 0x00020000);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
        const int j = c.j0 + 4 * tg + t;
        const bool ok = c.item >= 0 && j < c.M;
        p[tg] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(pr, ok ? (uint32_t)(c.s0 + j) * 4u : S4_OOB, 0, 0);
    }
}

// Byte offset of the activation row of this lane's token in group tg of
// cursor c's pass, or S4_OOB when there is no such token.
template <bool GATE_UP>
__device__ __forceinline__ uint32_t s4_xrow(const FfnArgs& a, const S4Cursor& c, int tg, uint32_t pair)
{
    const int j = c.j0 + 4 * tg + (lane_id() & 3);
    const bool ok = c.item >= 0 && j < c.M;
    uint32_t row;
    if constexpr (GATE_UP)
        row = (pair / (uint32_t)a.k) * (uint32_t)a.H * 2u;
    else
        row = (uint32_t)(c.s0 + j) * (uint32_t)a.I * 2u;
    return ok ? row : S4_OOB;
}

// Issue chunk c's loads into b.  Past-the-end cursors and K-blocks past the
// row read zeros through the buffer range checks, so every step issues the
// same loads with no branch.
template <int TG, bool GATE_UP>
__device__ __forceinline__ void s4_fetch(const FfnArgs& a, const S4Cursor& c, const uint32_t (&xrow)[TG], int K,
                                         S4Buf<TG>& b)
{
    const int lane = lane_id(), blk = lane >> 2;
    const int R = GATE_UP ? 2 * a.I : a.H;  // weight rows per expert
    const int nkb = K / 32;
    const bool live = c.item >= 0;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.w) + (size_t)c.e * R * (K / 2)), (short)0,
        live ? R * (K / 2) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.w_scale + (size_t)c.e * R * nkb), (short)0, live ? R * nkb : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(GATE_UP ? a.x : a.a_rows), (short)0,
        GATE_UP ? a.T * a.H * 2 : a.T * a.k * a.I * 2, 0x00020000);
    const int kb = c.kc / 32 + blk;  // this lane's K-block
    const bool kin = kb < nkb;
    {  // packed order: chunk cc of item it is [group][lane][16 B], its scales [lane][8 B]
        const int cc = c.kc / S4_KC, nb = min(S4_KB, nkb - S4_KB * cc);
        const uint32_t wb = (uint32_t)c.it * 512u * nkb + (uint32_t)cc * 8192u + 16u * lane;
#pragma unroll
        for (int g = 0; g < S4_RG; ++g)
            b.w[g] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   wr, kin ? wb + (uint32_t)(64 * nb * g) : S4_OOB, 0, 2));
        const uint32_t sb = (uint32_t)c.it * 32u * nkb + (uint32_t)cc * 512u + 8u * lane;
        const uint2 sv = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sr, kin ? sb : S4_OOB, 0, 2));
        b.s[0] = sv.x;
        b.s[1] = sv.y;
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
        const uint32_t xo = kin ? xrow[tg] + 64u * kb : S4_OOB;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            b.x[tg][q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 16u * q, 0, 0));
    }
}

// Byte SEL of q (two E2M1 codes, low nibble first) times scale, as two bf16.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4_pair(uint32_t q, float scale)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, SEL));
}

// Multiply one chunk into the token groups' accumulators; groups after the
// first only when `all` (a pass with at most 4 tokens skips them).  The E2M1
// codes are decoded once per K step and feed every group.
template <int TG>
__device__ __forceinline__ void s4_compute(const S4Buf<TG>& b, bool all, f32x4 (&acc)[TG][S4_RG])
{
    float sc[S4_RG];
#pragma unroll
    for (int g = 0; g < S4_RG; ++g)
        sc[g] = e8m0_to_f32((b.s[g / 4] >> (8 * (g % 4))) & 0xFFu);
#pragma unroll
    for (int s = 0; s < 8; ++s) {  // 4 K per step: codes 4s..4s+3 = bytes 2s, 2s+1 of the lane's 16
        uint32_t x0[TG], x1[TG];
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
            const u32x4 xv = b.x[tg][s / 2];
            x0[tg] = (s & 1) ? xv.z : xv.x;
            x1[tg] = (s & 1) ? xv.w : xv.y;
        }
        uint32_t a0[S4_RG], a1[S4_RG];
#pragma unroll
        for (int g = 0; g < S4_RG; ++g) {
            const uint32_t q = b.w[g][s / 2];
            a0[g] = (s & 1) ? cvt_fp4_pair<2>(q, sc[g]) : cvt_fp4_pair<0>(q, sc[g]);
            a1[g] = (s & 1) ? cvt_fp4_pair<3>(q, sc[g]) : cvt_fp4_pair<1>(q, sc[g]);
            acc[0][g] = mfma4(a0[g], a1[g], x0[0], x1[0], acc[0][g]);
        }
        if (TG > 1 && all) {
#pragma unroll
            for (int tg = 1; tg < TG; ++tg)
#pragma unroll
                for (int g = 0; g < S4_RG; ++g) acc[tg][g] = mfma4(a0[g], a1[g], x0[tg], x1[tg], acc[tg][g]);
        }
        __builtin_amdgcn_sched_barrier(0);  // decode one K step at a time (hoisting them all spills)
    }
}

// One step of the cross-block sum: keep v[0 .. 16>>J) (the half selected by
// bit J of this lane's block) and add the partner block's copies of it.
template <int J>
__device__ __forceinline__ void s4_halve(float (&v)[32], int blk)
{
    constexpr int half = 16 >> J;
    const bool hi = (blk >> J) & 1;
#pragma unroll
    for (int ci = 0; ci < half; ++ci) {
        const float send = hi ? v[ci] : v[ci + half];
        const float keep = hi ? v[ci + half] : v[ci];
        v[ci] = keep + __shfl_xor(send, 4 << J, WAVE);
    }
}

// Sum the 16 blocks' partials of token group tg and write its outputs.  v[ci]
// stands for item row i(ci); every step keeps half of the values and adds the
// partner lane's copies, so after 4 steps lane (b, t) holds two rows summed
// over all blocks: gate/up: gate row n and up row n with n = bitrev4(b);
// down: rows 2*bitrev4(b) and 2*bitrev4(b)+1.
template <bool GATE_UP>
__device__ __forceinline__ void s4_epilogue(const FfnArgs& a, const S4Cursor& c, int tg, f32x4 (&acc)[S4_RG])
{
    const int lane = lane_id(), blk = lane >> 2, t = lane & 3;
    float v[32];
#pragma unroll
    for (int ci = 0; ci < 32; ++ci) {
        // index bits from low: gate/up [row bit 4, row bits 0..3]; down [row bits 0..4]
        const int i = GATE_UP ? (((ci >> 1) & 15) | ((ci & 1) << 4)) : ci;
        v[ci] = acc[i / 4][i % 4];
    }
    s4_halve<0>(v, blk);
    s4_halve<1>(v, blk);
    s4_halve<2>(v, blk);
    s4_halve<3>(v, blk);
    const int rb = ((blk & 1) << 3) | ((blk & 2) << 1) | ((blk & 4) >> 1) | ((blk & 8) >> 3);  // bitrev4(blk)
    const int j = c.j0 + 4 * tg + t;
    if (j < c.M) {
        if constexpr (GATE_UP) {
            a.out[(size_t)(c.s0 + j) * a.I + 16 * c.it + rb] = (uint16_t)f32_to_bf16(silu(v[0]) * v[1]);
        } else {
            *reinterpret_cast<uint32_t*>(a.out + (size_t)(c.s0 + j) * a.H + 32 * c.it + 2 * rb) =
                pack_bf16x2(v[0], v[1]);
        }
    }
#pragma unroll
    for (int g = 0; g < S4_RG; ++g) acc[g] = f32x4{0, 0, 0, 0};
}

// One pipeline step: fetch cursor c1's chunk into nxt while multiplying c0's
// (in cur), and finish c0's pass if c1 starts another.  p holds c1's pair
// indices (loaded one step ago) and receives c2's.
template <int TG, bool GATE_UP>
__device__ __forceinline__ void s4_step(const FfnArgs& a, const S4Experts& x, int K, int n_items, int tiles, int nw,
                                        S4Cursor& c0, S4Cursor& c1, uint32_t (&p)[TG], S4Buf<TG>& cur,
                                        S4Buf<TG>& nxt, f32x4 (&acc)[TG][S4_RG])
{
    uint32_t xrow[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) xrow[tg] = s4_xrow<GATE_UP>(a, c1, tg, p[tg]);
    const S4Cursor c2 = s4_next<TG>(x, c1, K, n_items, tiles, nw);
    if constexpr (GATE_UP) s4_pairs<TG>(a, c2, p);
    s4_fetch<TG, GATE_UP>(a, c1, xrow, K, nxt);
    // groups past the pass's last token are loaded (as zeros) but not multiplied
    const bool all_groups = TG == 1 || c0.M - c0.j0 > 4 * (TG - 1);
    s4_compute<TG>(cur, all_groups, acc);
    if (c1.item != c0.item || c1.j0 != c0.j0) {
        mfma_drain();
        s4_epilogue<GATE_UP>(a, c0, 0, acc[0]);
        if (all_groups)
#pragma unroll
            for (int tg = 1; tg < TG; ++tg) s4_epilogue<GATE_UP>(a, c0, tg, acc[tg]);
    }
    c0 = c1;
    c1 = c2;
}

// Persistent over items (item = touched expert x 32-row tile; gate/up N = I,
// K = H; down N = H, K = I); wave w takes items w, w + nw, ...  gate/up: all
// resident waves, numbered block by block (the 4 waves of a block stream
// neighbouring rows).  down: the items are dealt out in equal rounds -- with
// R rounds of the resident waves needed, only ceil(items / R) waves take part
// and the rest exit, so that no short last round runs on a fraction of the
// waves; these are numbered across blocks first, to spread them over all
// CUs.  (Measured on the 20b decode shapes: each choice is the faster one for
// its projection.)
template <int TG, bool GATE_UP>
__global__ __launch_bounds__(S4_THREADS, 2) void skinny4_kernel(FfnArgs a)
{
    const int K = GATE_UP ? a.H : a.I;
    const int tiles = GATE_UP ? a.I / 16 : a.H / 32;
    const S4Experts x = s4_experts(a);
    const int n_items = x.active * tiles;
    const int nw_all = gridDim.x * S4_WPB;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);  // uniform per wave
    int nw = nw_all, w = blockIdx.x * S4_WPB + wave;
    if constexpr (!GATE_UP) {
        const int rounds = (n_items + nw_all - 1) / nw_all;
        nw = rounds > 0 ? (n_items + rounds - 1) / rounds : 1;
        w = wave * gridDim.x + blockIdx.x;
        if (w >= nw) return;
    }
    S4Cursor c0 = s4_item(x, w, n_items, tiles);
    if (c0.item < 0) return;  // uniform per wave

    S4Buf<TG> b0, b1;
    uint32_t p[TG], xrow[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) p[tg] = 0u;
    if constexpr (GATE_UP) s4_pairs<TG>(a, c0, p);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) xrow[tg] = s4_xrow<GATE_UP>(a, c0, tg, p[tg]);
    s4_fetch<TG, GATE_UP>(a, c0, xrow, K, b0);
    S4Cursor c1 = s4_next<TG>(x, c0, K, n_items, tiles, nw);
    if constexpr (GATE_UP) s4_pairs<TG>(a, c1, p);
    f32x4 acc[TG][S4_RG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
        for (int g = 0; g < S4_RG; ++g) acc[tg][g] = f32x4{0, 0, 0, 0};
    while (true) {  // two steps per iteration so the buffers swap roles without copies
        s4_step<TG, GATE_UP>(a, x, K, n_items, tiles, nw, c0, c1, p, b0, b1, acc);
        if (c0.item < 0) break;
        s4_step<TG, GATE_UP>(a, x, K, n_items, tiles, nw, c0, c1, p, b1, b0, acc);
        if (c0.item < 0) break;
    }
}

bool skinny4_supported(const FfnArgs& a)
{
    // 32-bit buffer offsets: one expert's weights, the activations and the
    // pair list must each stay below 2^31 bytes
    const long long lim = 1ll << 31;
    const long long P = (long long)a.T * a.k;
    return (long long)a.I * a.H < lim && (long long)a.T * a.H * 2 < lim && P * a.I * 2 < lim && P * 4 < lim;
}

template <int TG, bool GATE_UP>
static hipError_t launch_skinny4_tg(const FfnArgs& a, hipStream_t s)
{
    static const int cap = resident_blocks(reinterpret_cast<const void*>(&skinny4_kernel<TG, GATE_UP>), S4_THREADS);
    const int P = a.T * a.k;
    const int tiles = GATE_UP ? a.I / 16 : a.H / 32;
    const long long waves = (long long)(P < a.E ? P : a.E) * tiles;
    const long long blocks = (waves + S4_WPB - 1) / S4_WPB;
    const int grid = (int)(blocks < cap ? blocks : cap);
    hipLaunchKernelGGL((skinny4_kernel<TG, GATE_UP>), dim3(grid), dim3(S4_THREADS), 0, s, a);
    return hipGetLastError();
}

// An expert sees at most T tokens: one 4-token group covers T <= 4, else two
// groups (8 tokens per pass over the weights).
template <bool GATE_UP>
static hipError_t launch_skinny4(const FfnArgs& a, hipStream_t s)
{
    return a.T <= 4 ? launch_skinny4_tg<1, GATE_UP>(a, s) : launch_skinny4_tg<2, GATE_UP>(a, s);
}

hipError_t launch_gate_up_skinny(const FfnArgs& a, hipStream_t s)
{
    if (a.wfmt == 2) return launch_skinny4<true>(a, s);
    return a.wfmt == 0 ? launch_skinny<0, true>(a, s) : launch_skinny<1, true>(a, s);
}

hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t s)
{
    if (a.wfmt == 2) return launch_skinny4<false>(a, s);
    return a.wfmt == 0 ? launch_skinny<0, false>(a, s) : launch_skinny<1, false>(a, s);
}

}  // namespace moe
