// Backward of the MoE layer: the training variant (full-parameter fine-tuning:
// "kappa-20b-131k" model card; bf16 forward with fp32 accumulation, and
// activations recomputed during backprop instead of stored: "Persona Kappa:
// training a 20B LLM on desktop GPUs", section "Techniques That Made It
// Fit").  The entry point recomputes the forward, keeping g and u.  Given
// dy = dL/dy, per pair (token t, slot j, expert e) of the forward
//   dw_j = dy . o_j,   do_j = w_j dy,   da = Wd^T do_j,
//   dg = da * u * silu'(g),  du = da * silu(g),
//   dx += Wg^T dg + Wu^T du,   dWd[e] += do_j a^T,   dWgu[e] += [dg; du] x^T,
// and per token, through the softmax over the k selected logits,
//   dl_j = w_j (dw_j - sum_i w_i dw_i),  dx += sum_j dl_j Wr[e_j],  dWr[e_j] += dl_j x.
//
// Every contraction runs as an "NT" product (both operands contiguous along
// the contracted index) on bf16 MFMA with fp32 accumulation:
//   - the data gradients da and dx_pair contract over a weight's row index,
//     so they use the forward's tiled down-projection kernel on transposed
//     copies of W_down and W_gate_up (transpose_batched_kernel);
//   - the weight gradients contract over an expert's tokens, so the sorted
//     activation rows of each expert segment are transposed into a
//     zero-padded [rows][Kpad_e] block (transpose_segments_kernel, Kpad_e =
//     segment length rounded up to 64) and the tiled kernel's weight-gradient
//     mode multiplies them per expert.
// Everything else (combine backward, SwiGLU backward, router backward and dx)
// is elementwise or a row reduction.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// ------------------------------------------------------------------ transposes

constexpr int TR_TILE = 64;              // 64 x 64 element tiles
constexpr int TR_LD = TR_TILE + 8;       // LDS row stride (bf16)
constexpr int TR_THREADS = 256;

// Transpose one 64 x 64 tile through LDS.  in_row(i) gives the source row of
// tile row i (or null: the row reads as zeros); source columns c0.. (C
// columns per row, multiple of 8).  out_row(c) gives the destination row of
// tile column c (or null: skipped); it receives tile rows 0..nr-1 (nr a
// multiple of 8) at element offsets 0..nr-1.
template <typename InRow, typename OutRow>
__device__ __forceinline__ void transpose_tile(InRow in_row, int c0, int C, OutRow out_row, int nr, uint16_t* tile)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int v = t + TR_THREADS * q;  // 512 vectors of 8 columns
        const int i = v >> 3, cv = (v & 7) * 8;
        const uint16_t* src = in_row(i);
        u32x4 d = u32x4{0, 0, 0, 0};
        if (src && c0 + cv < C) d = *reinterpret_cast<const u32x4*>(src + c0 + cv);
        *reinterpret_cast<u32x4*>(tile + i * TR_LD + cv) = d;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int v = t + TR_THREADS * q;  // 512 output vectors of 8 rows
        const int c = v >> 3, iv = (v & 7) * 8;
        uint16_t* dst = out_row(c);
        if (!dst || iv >= nr) continue;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            w[p] = (uint32_t)tile[(iv + 2 * p) * TR_LD + c] | ((uint32_t)tile[(iv + 2 * p + 1) * TR_LD + c] << 16);
        *reinterpret_cast<u32x4*>(dst + iv) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// out[b][c][r] = in[b][r][c] for b < nb (grid.z), r < R, c < C (R, C multiples of 8).
__global__ __launch_bounds__(TR_THREADS) void transpose_batched_kernel(const uint16_t* __restrict__ in,
                                                                      uint16_t* __restrict__ out, int R, int C)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[TR_TILE * TR_LD];
    const size_t b = blockIdx.z;
    const int r0 = blockIdx.x * TR_TILE, c0 = blockIdx.y * TR_TILE;
    const uint16_t* ib = in + b * R * C;
    uint16_t* ob = out + b * R * C;
    const int nr = min(TR_TILE, R - r0);
    transpose_tile([&](int i) { return r0 + i < R ? ib + (size_t)(r0 + i) * C : nullptr; }, c0, C,
                   [&](int c) { return c0 + c < C ? ob + (size_t)(c0 + c) * R + r0 : nullptr; }, nr, tile);
}

// Per expert segment e (Kpad_e = padoff[e+1] - padoff[e]): out block at
// C * padoff[e], [C][Kpad_e], with out[c][j] = src(e, j)[c] for j < M_e and 0
// for M_e <= j < Kpad_e.  src(e, j) is row off[e] + j of `in` (rows of C
// elements), or with GATHER the token row sorted_pairs[off[e] + j] / k.
template <bool GATHER>
__global__ __launch_bounds__(TR_THREADS) void transpose_segments_kernel(const uint16_t* __restrict__ in, int C,
                                                                       const int32_t* __restrict__ offsets,
                                                                       const int32_t* __restrict__ padoff,
                                                                       const int32_t* __restrict__ sorted_pairs,
                                                                       int k, int E, uint16_t* __restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[TR_TILE * TR_LD];
    __shared__ int rows[TR_TILE];
    int jt = 0;
    const int e = locate_m_tile(offsets, E, TR_TILE, blockIdx.x, &jt);  // every wave computes the same
    if (e < 0) return;  // uniform: past the last tile
    const int s0 = offsets[e], M = offsets[e + 1] - s0;
    const int p0 = padoff[e], Kpad = padoff[e + 1] - p0;
    const int j0 = jt * TR_TILE;
    const int c0 = blockIdx.y * TR_TILE;
    if (threadIdx.x < TR_TILE) {
        const int j = j0 + threadIdx.x;
        rows[threadIdx.x] = j < M ? (GATHER ? sorted_pairs[s0 + j] / k : s0 + j) : -1;
    }
    __syncthreads();
    uint16_t* ob = out + (size_t)C * p0;
    transpose_tile([&](int i) { return rows[i] >= 0 ? in + (size_t)rows[i] * C : nullptr; }, c0, C,
                   [&](int c) { return c0 + c < C ? ob + (size_t)(c0 + c) * Kpad + j0 : nullptr; },
                   min(TR_TILE, Kpad - j0), tile);
}

// Padded segment offsets: Kpad_e = ceil(M_e / 64) * 64, padoff [E+1] their
// exclusive prefix; also zeroes the padding entries of dlT (the router
// gradient per sorted position, written for real positions by
// router_bwd_kernel).  One wave.
__global__ __launch_bounds__(WAVE) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                          int32_t* __restrict__ padoff, uint16_t* __restrict__ dlT)
{
    const int lane = lane_id();
    int run = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane;
        const int M = e < E ? offsets[e + 1] - offsets[e] : 0;
        const int kp = (M + TR_TILE - 1) / TR_TILE * TR_TILE;
        const int ex = wave_excl_scan(kp) + run;
        if (e < E) {
            padoff[e] = ex;
            for (int j = M; j < kp; ++j) dlT[ex + j] = 0;
        }
        run = __shfl(ex + kp, WAVE - 1, WAVE);
    }
    if (lane == 0) padoff[E] = run;
}

// ------------------------------------------------------------------ router weight gradient
// dWr[e] = sum over expert e's sorted rows i (token t_i) of dl_i * x[t_i], in
// two passes that fix the order of every sum.  Pass 1: each expert segment is
// cut into splits of RW_ROWS consecutive sorted rows (the splits of all
// experts numbered in expert order, as locate_m_tile numbers M-tiles), and a
// workgroup sums its split's rows for RW_COLS hidden columns in row order, in
// fp32, into part[split][H].  Pass 2 adds an expert's splits in split order.
// dl_i is the bf16 value router_bwd_kernel wrote to dlT.
constexpr int RW_ROWS = 64;                 // sorted rows per split (one per lane of a wave)
constexpr int RW_THREADS = 256;
constexpr int RW_COLS = RW_THREADS * 4;     // hidden columns per workgroup, 4 per thread
constexpr int RW_BATCH = 16;                // row loads in flight per thread

__global__ __launch_bounds__(RW_THREADS) void router_wgrad_partial_kernel(
    int H, int E, int k, const int32_t* __restrict__ offsets, const int32_t* __restrict__ padoff,
    const int32_t* __restrict__ sorted_pairs, const uint16_t* __restrict__ dlT, const uint16_t* __restrict__ x,
    float* __restrict__ part)
{
    int mt;
    const int e = locate_m_tile(offsets, E, RW_ROWS, blockIdx.x, &mt);  // the same in every wave
    if (e < 0) return;  // uniform: past the last split
    const int r0 = mt * RW_ROWS;
    const int n = min(RW_ROWS, offsets[e + 1] - offsets[e] - r0);
    const int lane = lane_id();
    int tok = 0;
    float dl = 0.f;
    if (lane < n) {
        tok = sorted_pairs[offsets[e] + r0 + lane] / k;
        dl = bf16_to_f32(dlT[padoff[e] + r0 + lane]);
    }
    const int h = blockIdx.y * RW_COLS + threadIdx.x * 4;  // H % 32 == 0: all 4 columns or none
    const bool col_ok = h < H;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < n; i0 += RW_BATCH) {
        uint2 v[RW_BATCH];
#pragma unroll
        for (int i = 0; i < RW_BATCH; ++i) {
            const int t = __builtin_amdgcn_readlane(tok, i0 + i);
            v[i] = (col_ok && i0 + i < n) ? *reinterpret_cast<const uint2*>(x + (size_t)t * H + h) : uint2{0, 0};
        }
#pragma unroll
        for (int i = 0; i < RW_BATCH; ++i) {
            if (i0 + i < n) {  // uniform
                const float d = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(dl), i0 + i));
                acc[0] = fmaf(d, bf16_lo(v[i].x), acc[0]);
                acc[1] = fmaf(d, bf16_hi(v[i].x), acc[1]);
                acc[2] = fmaf(d, bf16_lo(v[i].y), acc[2]);
                acc[3] = fmaf(d, bf16_hi(v[i].y), acc[3]);
            }
        }
    }
    if (col_ok) *reinterpret_cast<float4*>(part + (size_t)blockIdx.x * H + h) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// Pass 2: one thread per (expert, column); an expert without rows gets zeros.
__global__ __launch_bounds__(RW_THREADS) void router_wgrad_reduce_kernel(int H, int E,
                                                                         const int32_t* __restrict__ offsets,
                                                                         const float* __restrict__ part,
                                                                         float* __restrict__ dwr)
{
    __shared__ int first_split, n_splits;
    const int e = blockIdx.y;
    if (threadIdx.x < WAVE) {
        const int lane = lane_id();
        int before = 0;
        for (int base = 0; base < e; base += WAVE) {
            const int j = base + lane;
            const int c = j < e ? (offsets[j + 1] - offsets[j] + RW_ROWS - 1) / RW_ROWS : 0;
            before += wave_sum(c);
        }
        if (lane == 0) {
            first_split = before;
            n_splits = (offsets[e + 1] - offsets[e] + RW_ROWS - 1) / RW_ROWS;
        }
    }
    __syncthreads();
    const int h = blockIdx.x * RW_THREADS + threadIdx.x;
    if (h >= H) return;
    const float* col = part + (size_t)first_split * H + h;
    float sum = 0.f;
    int j = 0;
    for (; j + 8 <= n_splits; j += 8) {  // 8 loads in flight, added in split order
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = col[(size_t)(j + q) * H];
#pragma unroll
        for (int q = 0; q < 8; ++q) sum += v[q];
    }
    for (; j < n_splits; ++j) sum += col[(size_t)j * H];
    dwr[(size_t)e * H + h] = sum;
}

// ------------------------------------------------------------------ elementwise / reductions

// Combine backward, one wave per sorted row s (pair p = sorted_pairs[s],
// token t = p / k): dO[s] = w_p * dy[t] (bf16), dw[p] = dy[t] . y_sorted[s].
__global__ __launch_bounds__(256) void combine_bwd_kernel(int P, int H, int k, const uint16_t* __restrict__ dy,
                                                         const uint16_t* __restrict__ ys,
                                                         const int32_t* __restrict__ sorted_pairs,
                                                         const float* __restrict__ topk_w,
                                                         uint16_t* __restrict__ dO, float* __restrict__ dw)
{
    const int s = (int)((blockIdx.x * blockDim.x + threadIdx.x) / WAVE);
    if (s >= P) return;
    const int lane = lane_id();
    const int p = sorted_pairs[s], tok = p / k;
    const float w = topk_w[p];
    const uint16_t* dyr = dy + (size_t)tok * H;
    const uint16_t* yr = ys + (size_t)s * H;
    uint16_t* dor = dO + (size_t)s * H;
    float dot = 0.0f;
    for (int c = 8 * lane; c < H; c += 8 * WAVE) {
        const u32x4 d = *reinterpret_cast<const u32x4*>(dyr + c);
        const u32x4 y = *reinterpret_cast<const u32x4*>(yr + c);
        const uint32_t dv[4] = {d.x, d.y, d.z, d.w}, yv[4] = {y.x, y.y, y.z, y.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float d0 = bf16_lo(dv[q]), d1 = bf16_hi(dv[q]);
            dot += d0 * bf16_lo(yv[q]) + d1 * bf16_hi(yv[q]);
            o[q] = pack_bf16x2(w * d0, w * d1);
        }
        *reinterpret_cast<u32x4*>(dor + c) = u32x4{o[0], o[1], o[2], o[3]};
    }
    dot = wave_sum(dot);
    if (lane == 0) dw[p] = dot;
}

// SwiGLU backward, 8 elements per thread: from da [P][I] and g, u ([P][2I]:
// g then u), dgu[s][i] = da * u * silu'(g), dgu[s][I + i] = da * silu(g).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(int P, int I, const uint16_t* __restrict__ da,
                                                        const uint16_t* __restrict__ gu, uint16_t* __restrict__ dgu)
{
    const long long v = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int per_row = I / 8;
    if (v >= (long long)P * per_row) return;
    const int s = (int)(v / per_row), i = (int)(v % per_row) * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(da + (size_t)s * I + i);
    const u32x4 g = *reinterpret_cast<const u32x4*>(gu + (size_t)s * 2 * I + i);
    const u32x4 u = *reinterpret_cast<const u32x4*>(gu + (size_t)s * 2 * I + I + i);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
    uint32_t dg[4], du[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float r[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float x = h ? bf16_hi(gv[q]) : bf16_lo(gv[q]);
            const float up = h ? bf16_hi(uv[q]) : bf16_lo(uv[q]);
            const float d = h ? bf16_hi(av[q]) : bf16_lo(av[q]);
            const float sg = 1.0f / (1.0f + __expf(-x));
            r[0][h] = d * up * sg * (1.0f + x * (1.0f - sg));
            r[1][h] = d * x * sg;
        }
        dg[q] = pack_bf16x2(r[0][0], r[0][1]);
        du[q] = pack_bf16x2(r[1][0], r[1][1]);
    }
    *reinterpret_cast<u32x4*>(dgu + (size_t)s * 2 * I + i) = u32x4{dg[0], dg[1], dg[2], dg[3]};
    *reinterpret_cast<u32x4*>(dgu + (size_t)s * 2 * I + I + i) = u32x4{du[0], du[1], du[2], du[3]};
}

// Router backward and dx, one workgroup per token t:
//   dl_j = w_j (dw_j - sum_i w_i dw_i)      (written to dlT at the pair's padded sorted position)
//   dx[t] = sum_j dx_pair[rank(t, j)] + sum_j dl_j Wr[e_j]      (slot order)
__global__ __launch_bounds__(256) void router_bwd_kernel(int H, int k, const uint16_t* __restrict__ wr,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_w,
                                                        const float* __restrict__ dw,
                                                        const int32_t* __restrict__ pair_rank,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ padoff,
                                                        const uint16_t* __restrict__ dxp, uint16_t* __restrict__ dlT,
                                                        uint16_t* __restrict__ dx)
{
    const int tok = blockIdx.x;
    float dl[8];
    int ex[8], rk[8];
    float sbar = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) sbar += topk_w[(size_t)tok * k + j] * dw[(size_t)tok * k + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        dl[j] = 0.0f;
        ex[j] = 0;
        rk[j] = 0;
        if (j < k) {
            const size_t p = (size_t)tok * k + j;
            dl[j] = topk_w[p] * (dw[p] - sbar);
            ex[j] = topk_idx[p];
            rk[j] = pair_rank[p];
        }
    }
    if (threadIdx.x < k) {  // thread j writes slot j's dl at its padded sorted position
        const int j = threadIdx.x;
        float v = dl[0];
        int ej = ex[0], rj = rk[0];
#pragma unroll
        for (int q = 1; q < 8; ++q)
            if (q == j) {
                v = dl[q];
                ej = ex[q];
                rj = rk[q];
            }
        dlT[padoff[ej] + rj - offsets[ej]] = (uint16_t)f32_to_bf16(v);
    }
    for (int c = 8 * threadIdx.x; c < H; c += 8 * blockDim.x) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= k) continue;
            const u32x4 a = *reinterpret_cast<const u32x4*>(dxp + (size_t)rk[j] * H + c);
            const u32x4 w = *reinterpret_cast<const u32x4*>(wr + (size_t)ex[j] * H + c);
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf16_lo(av[q]) + dl[j] * bf16_lo(wv[q]);
                acc[2 * q + 1] += bf16_hi(av[q]) + dl[j] * bf16_hi(wv[q]);
            }
        }
        *reinterpret_cast<u32x4*>(dx + (size_t)tok * H + c) =
            u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                  pack_bf16x2(acc[6], acc[7])};
    }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, long long n)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ------------------------------------------------------------------ launchers

hipError_t launch_zero_f32(float* p, long long n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_transpose_batched(const uint16_t* in, uint16_t* out, int nb, int R, int C, hipStream_t s)
{
    const dim3 grid((R + TR_TILE - 1) / TR_TILE, (C + TR_TILE - 1) / TR_TILE, nb);
    hipLaunchKernelGGL(transpose_batched_kernel, grid, dim3(TR_THREADS), 0, s, in, out, R, C);
    return hipGetLastError();
}

int backward_pad_rows(int P, int E) { return P + (TR_TILE - 1) * E; }

// sum over experts of ceil(M_e / RW_ROWS) <= floor((P + (RW_ROWS - 1) E) / RW_ROWS)
long long router_wgrad_splits(int P, int E) { return ((long long)P + (long long)(RW_ROWS - 1) * E) / RW_ROWS; }

hipError_t launch_router_wgrad(int H, int E, int k, int P, const int32_t* offsets, const int32_t* padoff,
                               const int32_t* sorted_pairs, const uint16_t* dlT, const uint16_t* x, float* part,
                               float* dwr, hipStream_t s)
{
    const long long ns = router_wgrad_splits(P, E);
    if (ns > 0) {
        const dim3 grid((unsigned)ns, (H + RW_COLS - 1) / RW_COLS);
        hipLaunchKernelGGL(router_wgrad_partial_kernel, grid, dim3(RW_THREADS), 0, s, H, E, k, offsets, padoff,
                           sorted_pairs, dlT, x, part);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const dim3 grid2((H + RW_THREADS - 1) / RW_THREADS, E);
    hipLaunchKernelGGL(router_wgrad_reduce_kernel, grid2, dim3(RW_THREADS), 0, s, H, E, offsets, part, dwr);
    return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* padoff, uint16_t* dlT, hipStream_t s)
{
    hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(WAVE), 0, s, offsets, E, padoff, dlT);
    return hipGetLastError();
}

hipError_t launch_transpose_segments(const uint16_t* in, int C, bool gather, const int32_t* offsets,
                                     const int32_t* padoff, const int32_t* sorted_pairs, int k, int P, int E,
                                     uint16_t* out, hipStream_t s)
{
    const dim3 grid((P + TR_TILE - 1) / TR_TILE + E, (C + TR_TILE - 1) / TR_TILE);
    if (gather)
        hipLaunchKernelGGL(transpose_segments_kernel<true>, grid, dim3(TR_THREADS), 0, s, in, C, offsets, padoff,
                           sorted_pairs, k, E, out);
    else
        hipLaunchKernelGGL(transpose_segments_kernel<false>, grid, dim3(TR_THREADS), 0, s, in, C, offsets, padoff,
                           sorted_pairs, k, E, out);
    return hipGetLastError();
}

hipError_t launch_combine_bwd(int P, int H, int k, const uint16_t* dy, const uint16_t* ys, const int32_t* sorted_pairs,
                              const float* topk_w, uint16_t* dO, float* dw, hipStream_t s)
{
    const int blocks = (P + 3) / 4;
    hipLaunchKernelGGL(combine_bwd_kernel, dim3(blocks), dim3(256), 0, s, P, H, k, dy, ys, sorted_pairs, topk_w, dO,
                       dw);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int P, int I, const uint16_t* da, const uint16_t* gu, uint16_t* dgu, hipStream_t s)
{
    const long long n = (long long)P * (I / 8);
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P, I, da, gu, dgu);
    return hipGetLastError();
}

hipError_t launch_router_bwd(int T, int H, int k, const uint16_t* wr, const int32_t* topk_idx, const float* topk_w,
                             const float* dw, const int32_t* pair_rank, const int32_t* offsets, const int32_t* padoff,
                             const uint16_t* dxp, uint16_t* dlT, uint16_t* dx, hipStream_t s)
{
    hipLaunchKernelGGL(router_bwd_kernel, dim3(T), dim3(256), 0, s, H, k, wr, topk_idx, topk_w, dw, pair_rank,
                       offsets, padoff, dxp, dlT, dx);
    return hipGetLastError();
}

}  // namespace moe
