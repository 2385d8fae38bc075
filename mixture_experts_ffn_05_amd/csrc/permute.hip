// Permutation of the (token, expert) pairs into expert-contiguous segments.
//
// A stable counting sort of pair ids p = t*k + j by expert (the pages leave
// the order open; stability makes the result unique, so it can be checked
// bit for bit).  Ranks inside a chunk of 1024 pairs come from wave ballots
// (lanes holding the same expert find each other bit by bit), so nothing
// depends on the order atomics land in.
//
//   P <= SMALL_P : one workgroup does histogram, scan and scatter.
//   otherwise    : count kernel (per-chunk ranks + per-chunk histograms),
//                  scan kernel (offsets + per-chunk bases), scatter kernel.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int PB_THREADS = PERMUTE_CHUNK;      // one pair per thread per pass
constexpr int PB_WAVES = PB_THREADS / WAVE;    // 16
constexpr int MAX_E = 256;
constexpr int SMALL_P = 4096;

// Stable rank of `key` among the earlier threads of the workgroup holding the
// same key (key < 0: no key).  wave_counts [PB_WAVES][E] must be zero on
// entry; chunk_total [E] receives the per-key counts of this pass.  Contains
// two barriers; every thread of the block must call it.
__device__ int block_stable_rank(int key, int E, int nbits, int* wave_counts, int* chunk_total)
{
    const int wave = threadIdx.x / WAVE;
    const bool valid = key >= 0;
    uint64_t peers = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((key >> b) & 1);
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    const int rank_in_wave = __popcll(peers & lanemask_lt());
    if (valid && rank_in_wave == 0) wave_counts[wave * E + key] = __popcll(peers);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = 0;
        for (int w = 0; w < PB_WAVES; ++w) {
            const int c = wave_counts[w * E + e];
            wave_counts[w * E + e] = run;
            run += c;
        }
        chunk_total[e] = run;
    }
    __syncthreads();
    return valid ? wave_counts[wave * E + key] + rank_in_wave : -1;
}

__device__ __forceinline__ int key_bits(int E) { return E <= 1 ? 0 : 32 - __clz(E - 1); }

// Exclusive scan of counts[0..E) in place by wave 0; offsets (global) gets the
// same values plus offsets[E] = total.
__device__ void scan_counts_wave0(int* counts, int E, int32_t* offsets)
{
    if (threadIdx.x >= WAVE) return;
    const int lane = lane_id();
    int run = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane;
        const int c = e < E ? counts[e] : 0;
        const int ex = wave_excl_scan(c) + run;
        if (e < E) {
            counts[e] = ex;
            offsets[e] = ex;
        }
        run = __shfl(ex + c, WAVE - 1, WAVE);
    }
    if (lane == 0) offsets[E] = run;
}

// Permutation of P <= 64 pairs by one wave, lane p holding pair p: stable
// ranks among equal experts from ballots, per-expert counts through LDS
// (counts [E]), then their exclusive scan.  No barrier: LDS accesses of one
// wave complete in order.
__device__ void permute_wave(int P, int E, const int32_t* __restrict__ topk_idx, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_rank, int* counts)
{
    const int lane = lane_id();
    const int key = lane < P ? topk_idx[lane] : -1;
    for (int e = lane; e < E; e += WAVE) counts[e] = 0;
    const bool valid = key >= 0;
    uint64_t peers = ballot(valid);
    const int nbits = key_bits(E);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((key >> b) & 1);
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lanemask_lt());
    if (valid && rank == 0) counts[key] = __popcll(peers);
    int run = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane;
        const int c = e < E ? counts[e] : 0;
        const int ex = wave_excl_scan(c) + run;
        if (e < E) {
            counts[e] = ex;
            offsets[e] = ex;
        }
        run = __shfl(ex + c, WAVE - 1, WAVE);
    }
    if (lane == 0) offsets[E] = run;
    if (valid) {
        const int s = counts[key] + rank;
        sorted_pairs[s] = lane;
        pair_rank[lane] = s;
    }
}

// Whole permutation of P <= SMALL_P pairs by one workgroup of PB_THREADS:
// histogram, exclusive scan, then the stable scatter in passes of 1024 pairs
// (at most 64 pairs: one wave, see permute_wave).
__device__ void permute_block(int P, int E, const int32_t* __restrict__ topk_idx, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_rank)
{
    __shared__ int wave_counts[PB_WAVES * MAX_E];
    __shared__ int chunk_total[MAX_E];
    __shared__ int cursor[MAX_E];
    if (P <= WAVE) {  // uniform
        if (threadIdx.x < WAVE) permute_wave(P, E, topk_idx, offsets, sorted_pairs, pair_rank, cursor);
        return;
    }
    const int nbits = key_bits(E);
    for (int e = threadIdx.x; e < E; e += blockDim.x) cursor[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) atomicAdd(&cursor[topk_idx[p]], 1);
    __syncthreads();
    scan_counts_wave0(cursor, E, offsets);
    __syncthreads();
    for (int c0 = 0; c0 < P; c0 += PB_THREADS) {
        for (int i = threadIdx.x; i < PB_WAVES * E; i += blockDim.x) wave_counts[i] = 0;
        __syncthreads();
        const int p = c0 + threadIdx.x;
        const int key = p < P ? topk_idx[p] : -1;
        const int r = block_stable_rank(key, E, nbits, wave_counts, chunk_total);
        if (key >= 0) {
            const int s = cursor[key] + r;
            sorted_pairs[s] = p;
            pair_rank[p] = s;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += blockDim.x) cursor[e] += chunk_total[e];
        __syncthreads();
    }
}

__global__ __launch_bounds__(PB_THREADS) void permute_small_kernel(int P, int E, const int32_t* __restrict__ topk_idx,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ sorted_pairs,
                                                                    int32_t* __restrict__ pair_rank)
{
    permute_block(P, E, topk_idx, offsets, sorted_pairs, pair_rank);
}

// Small batches: top-k selection of every token (one wave per token, logits
// [T][E] from the router) followed by the permutation, in one workgroup.  The
// selected experts also go to LDS, where the permutation reads them.
__global__ __launch_bounds__(PB_THREADS) void select_permute_small_kernel(
    int T, int E, int k, const double* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_rank)
{
    __shared__ int32_t keys[SMALL_P];
    for (int t = threadIdx.x / WAVE; t < T; t += PB_WAVES) {
        int32_t* idx = topk_idx + (size_t)t * k;
        if (E <= WAVE) {
            const int slot = wave_topk_softmax_rank(logits + (size_t)t * E, E, k, idx, topk_w + (size_t)t * k);
            if (slot >= 0) keys[t * k + slot] = (int32_t)lane_id();
        } else {
            const int ex = wave_topk_softmax(logits + (size_t)t * E, E, k, idx, topk_w + (size_t)t * k);
            if (ex >= 0) keys[t * k + lane_id()] = ex;
        }
    }
    __syncthreads();
    permute_block(T * k, E, keys, offsets, sorted_pairs, pair_rank);
}

// Pass 1 of the multi-block path: chunk b = blockIdx.x ranks its pairs and
// writes rank[p] and hist[b][e].
__global__ __launch_bounds__(PB_THREADS) void permute_count_kernel(int P, int E, const int32_t* __restrict__ topk_idx,
                                                                    int32_t* __restrict__ rank,
                                                                    int32_t* __restrict__ hist)
{
    __shared__ int wave_counts[PB_WAVES * MAX_E];
    __shared__ int chunk_total[MAX_E];
    for (int i = threadIdx.x; i < PB_WAVES * E; i += blockDim.x) wave_counts[i] = 0;
    __syncthreads();
    const int p = blockIdx.x * PB_THREADS + threadIdx.x;
    const int key = p < P ? topk_idx[p] : -1;
    const int r = block_stable_rank(key, E, key_bits(E), wave_counts, chunk_total);
    if (key >= 0) rank[p] = r;
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = chunk_total[e];
}

// Pass 2: per expert (one wave each), the exclusive prefix over chunks; then
// the expert offsets; hist[b][e] becomes the global base of chunk b inside
// expert e.
__global__ __launch_bounds__(PB_THREADS) void permute_scan_kernel(int nchunks, int E, int32_t* __restrict__ hist,
                                                                  int32_t* __restrict__ offsets)
{
    __shared__ int totals[MAX_E];
    const int wave = threadIdx.x / WAVE, lane = lane_id();
    for (int e = wave; e < E; e += PB_WAVES) {
        int run = 0;
        for (int b0 = 0; b0 < nchunks; b0 += WAVE) {
            const int b = b0 + lane;
            const int c = b < nchunks ? hist[(size_t)b * E + e] : 0;
            const int ex = wave_excl_scan(c) + run;
            if (b < nchunks) hist[(size_t)b * E + e] = ex;
            run = __shfl(ex + c, WAVE - 1, WAVE);
        }
        if (lane == 0) totals[e] = run;
    }
    __syncthreads();
    scan_counts_wave0(totals, E, offsets);
    __syncthreads();
    for (int i = threadIdx.x; i < nchunks * E; i += blockDim.x) hist[i] += totals[i % E];
}

// Pass 3: scatter.
__global__ __launch_bounds__(256) void permute_scatter_kernel(int P, int E, const int32_t* __restrict__ topk_idx,
                                                              const int32_t* __restrict__ rank,
                                                              const int32_t* __restrict__ hist,
                                                              int32_t* __restrict__ sorted_pairs,
                                                              int32_t* __restrict__ pair_rank)
{
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    const int e = topk_idx[p];
    const int s = hist[(size_t)(p / PB_THREADS) * E + e] + rank[p];
    sorted_pairs[s] = p;
    pair_rank[p] = s;
}

bool permute_fits_one_block(int P) { return P <= SMALL_P; }

hipError_t launch_select_permute_small(int T, int E, int k, const double* logits, int32_t* topk_idx, float* topk_w,
                                       int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_rank, hipStream_t s)
{
    hipLaunchKernelGGL(select_permute_small_kernel, dim3(1), dim3(PB_THREADS), 0, s, T, E, k, logits, topk_idx,
                       topk_w, offsets, sorted_pairs, pair_rank);
    return hipGetLastError();
}

size_t permute_scratch_bytes(int64_t P, int E)
{
    const int64_t nchunks = (P + PB_THREADS - 1) / PB_THREADS;
    return (size_t)(P + nchunks * E) * sizeof(int32_t);
}

hipError_t launch_permute(int P, int E, const int32_t* topk_idx, int32_t* offsets, int32_t* sorted_pairs,
                          int32_t* pair_rank, void* scratch, hipStream_t s)
{
    if (P <= SMALL_P) {
        hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(PB_THREADS), 0, s, P, E, topk_idx, offsets,
                           sorted_pairs, pair_rank);
        return hipGetLastError();
    }
    const int nchunks = (P + PB_THREADS - 1) / PB_THREADS;
    int32_t* rank = static_cast<int32_t*>(scratch);
    int32_t* hist = rank + P;
    hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(PB_THREADS), 0, s, P, E, topk_idx, rank, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(PB_THREADS), 0, s, nchunks, E, hist, offsets);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((P + 255) / 256), dim3(256), 0, s, P, E, topk_idx, rank, hist,
                       sorted_pairs, pair_rank);
    return hipGetLastError();
}

}  // namespace moe
