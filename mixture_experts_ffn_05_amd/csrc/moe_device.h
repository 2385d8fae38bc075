// Device-side helpers shared by the gfx950 kernels of the MoE FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;  // MFMA A/B operand (8 bf16 per lane)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;     // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // 16 raw bytes

constexpr int WAVE = 64;

// --------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even float -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16); }

// low / high bf16 of a packed pair, widened
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// --------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: D[16][16] += A[16][32] * B[32][16].
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each with the
// 8 K-values of group (l / 16); it receives D rows 4*(l/16) .. +3 of column
// l % 16.  Any K ordering works as long as A and B use the same one.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Idle cycles between the last MFMA of a K loop and the first read of its
// accumulator.  hipcc's hazard recognizer was seen to place no wait states
// before the first accumulator read in the block after a K loop
// (v_mfma_f32_16x16x32_bf16 on gfx950), so the read returned a stale partial
// sum.  Call it as the last statement of the loop body on the final
// iteration (the accumulator copies are materialised in the loop's exit
// block, after it).  20 wait states cover the 8-pass MFMA; the scheduling
// barriers keep the MFMAs from sinking below them.
__device__ __forceinline__ void mfma_drain()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// --------------------------------------------------------------- MXFP4
// Dequantise 8 E2M1 values (one 32-bit word, element 2i in the low nibble of
// byte i) times the block scale into 8 bf16 (exact: a power-of-two scale
// times a 2-significant-bit value).
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t q, float scale)
{
    u32x4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1));
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2));
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3));
    return r;
}

// E8M0 byte -> the float 2^(S-127) (S = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their
// no-wait maxima).
template <int n>
__device__ __forceinline__ void vm_wait()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// --------------------------------------------------------------- wave utils

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() { return (uint64_t(1) << lane_id()) - 1; }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Exclusive prefix sum of an int across the wave.
__device__ __forceinline__ int wave_excl_scan(int v)
{
    int lane = lane_id();
    int x = v;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        int y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    return x - v;
}

// The a-th (0-based) expert with a non-empty segment, found by one wave from
// expert_offsets [E+1].  Returns -1 if fewer than a+1 experts are non-empty.
__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ offsets, int E, int a)
{
    int lane = lane_id();
    for (int base = 0; base < E; base += WAVE) {
        int e = base + lane;
        bool act = e < E && offsets[e + 1] > offsets[e];
        uint64_t m = ballot(act);
        int cnt = __popcll(m);
        if (a < cnt) {
            int before = __popcll(m & lanemask_lt());
            uint64_t hit = ballot(act && before == a);
            return base + (int)__builtin_ctzll(hit);
        }
        a -= cnt;
    }
    return -1;
}

// Locate M-tile `tile` of the grouped schedule in which expert e owns
// ceil(M_e / BM) consecutive tiles.  One wave; returns the expert (or -1 when
// tile is past the end) and sets *mt to the tile index inside that expert.
__device__ __forceinline__ int locate_m_tile(const int32_t* __restrict__ offsets, int E, int BM, int tile, int* mt)
{
    int lane = lane_id();
    int before_chunk = 0;
    for (int base = 0; base < E; base += WAVE) {
        int e = base + lane;
        int n = 0;
        if (e < E) {
            int m = offsets[e + 1] - offsets[e];
            n = (m + BM - 1) / BM;
        }
        int excl = wave_excl_scan(n) + before_chunk;
        bool hit = (n > 0) && tile >= excl && tile < excl + n;
        uint64_t hm = ballot(hit);
        if (hm) {
            int src = (int)__builtin_ctzll(hm);
            int ex = __shfl(excl, src, WAVE);
            *mt = tile - ex;
            return base + src;
        }
        before_chunk = __shfl(excl + n, WAVE - 1, WAVE);
    }
    *mt = 0;
    return -1;
}

// --------------------------------------------------------------- routing
// Selection rule (the pages give top-k routing without a tie rule; the reading
// taken is): larger logit first, an exactly equal logit goes to the lower
// expert index; weights = softmax over the k selected logits.

// The value a logit is ranked and weighted by: a NaN logit (a NaN in the
// token's row or in the expert's router row) ranks below every number, as
// -infinity, so selection always yields k distinct experts in [0, E); a token
// whose logits are all NaN gets experts 0..k-1 by the tie rule and NaN
// weights.  (The pages say nothing of non-finite inputs; this is the reading
// taken.)
__device__ __forceinline__ double rank_key(double v) { return __builtin_isnan(v) ? -__builtin_inf() : v; }

// Does candidate (v, i) rank before (bv, bi)?  Larger logit first, then the
// lower expert index.
__device__ __forceinline__ bool ranks_before(double v, int i, double bv, int bi)
{
    return v > bv || (v == bv && i < bi);
}

// Lane l's value of v (l uniform), through two scalar lane reads.
__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Top-k for E <= 64 by one wave, lane e holding expert e: each lane counts
// the experts that rank before its own (larger logit, or equal logit and a
// lower index) over all E logits, read lane by lane from registers, so its
// rank is exact and the k lanes with rank < k own the slots -- no serial
// arg-max rounds.  Then the softmax over the k selected: each selected lane
// takes its own exp, and the sum runs in slot order exactly as
// wave_topk_softmax's does, so both give the same weights.  The lane of slot
// j writes slot j; returns this lane's slot, or -1.
__device__ __forceinline__ int wave_topk_softmax_rank(const double* row, int E, int k, int32_t* __restrict__ idx_out,
                                                      float* __restrict__ w_out)
{
    const int e = lane_id();
    const double v = e < E ? rank_key(row[e]) : -__builtin_inf();
    int rank = 0;
    for (int j = 0; j < E; ++j) rank += ranks_before(readlane_f64(v, j), j, v, e) ? 1 : 0;
    const bool sel = e < E && rank < k;
    const double v0 = readlane_f64(v, (int)__builtin_ctzll(ballot(sel && rank == 0)));
    const double ex = sel ? exp(v - v0) : 0.0;
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += readlane_f64(ex, (int)__builtin_ctzll(ballot(sel && rank == j)));
    if (sel) {
        idx_out[rank] = e;
        w_out[rank] = (float)(ex / z);
    }
    return sel ? rank : -1;
}

// Top-k of one token's E logits (row: global or LDS) by one wave: k rounds of
// a wave-wide arg-max (each lane owns experts lane, lane+64, ...), then the
// softmax over the k selected.  Lane j writes slot j and returns its expert
// (other lanes -1).
__device__ __forceinline__ int wave_topk_softmax(const double* row, int E, int k, int32_t* __restrict__ idx_out,
                                                 float* __restrict__ w_out)
{
    const int lane = lane_id();
    double v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + WAVE * i;
        v[i] = e < E ? rank_key(row[e]) : -__builtin_inf();
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
    int mine = -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < k && lane == j) {
            idx_out[j] = sel_i[j];
            w_out[j] = (float)(exp(sel_v[j] - sel_v[0]) / z);
            mine = sel_i[j];
        }
    }
    return mine;
}

}  // namespace moe
