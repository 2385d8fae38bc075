// Tile schedule shared by the tiled (prefill) grouped-GEMM kernels: which
// expert segment and which (weight, token) tile a workgroup takes, and the
// weight row behind each tile row.
//
// Each expert segment of the permutation is an independent GEMM of its weight
// rows (N side) by its M_e token rows.  A tile is GM_BW weight rows x GM_BT
// token rows.  Expert e owns ceil(M_e / GM_BT) * nt consecutive tiles, where
// nt = ceil(output columns / tile columns); inside an expert the tiles run in
// bands of GM_BAND M-tiles, the M-tiles of one N-tile adjacent, so neighbouring
// tiles share token rows or weight rows.
#pragma once

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int GM_BT = 256;    // tokens per tile
constexpr int GM_BW = 256;    // weight rows per tile
// M-tiles per band of the bf16 kernel's tile order.  (Measured on the 8192-token
// Zipf prefill, interleaved repeats: 8 gives gate/up 1175 us and down 631 us
// against 1199 and 641 us with 4; 12 and 16 the same as 8, 2 slower.  The MX
// kernel, whose token tile is the larger operand, keeps bands of 4.)
constexpr int GM_BAND = 8;

// Workgroup barrier after this wave's LDS writes have completed.  It carries
// no memory fence: the direct-to-LDS loads still in flight belong to later
// stages and are waited for explicitly (vm_wait), and a fence here would make
// the compiler drain them.  The asm memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// Which expert and local tile a linear tile index belongs to.  Expert e owns
// ceil(M_e / BT) * nt consecutive tiles.  One wave; returns -1 past the end.
template <int BT = GM_BT>
__device__ __forceinline__ int gm_locate(const int32_t* __restrict__ offsets, int E, int nt, int tile, int* local,
                                         int* mtiles)
{
    const int lane = lane_id();
    int before = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane;
        int mt = 0;
        if (e < E) mt = (offsets[e + 1] - offsets[e] + BT - 1) / BT;
        const int n = mt * nt;
        const int excl = wave_excl_scan(n) + before;
        const uint64_t hm = ballot(n > 0 && tile >= excl && tile < excl + n);
        if (hm) {
            const int src = (int)__builtin_ctzll(hm);
            *local = tile - __shfl(excl, src, WAVE);
            *mtiles = __shfl(mt, src, WAVE);
            return base + src;
        }
        before = __shfl(excl + n, WAVE - 1, WAVE);
    }
    return -1;
}

template <int BT = GM_BT>
__device__ __forceinline__ int gm_total_tiles(const int32_t* __restrict__ offsets, int E, int nt)
{
    int n = 0;
    for (int base = 0; base < E; base += WAVE) {
        const int e = base + lane_id();
        const int mt = e < E ? (offsets[e + 1] - offsets[e] + BT - 1) / BT : 0;
        n += wave_sum(mt);
    }
    return n * nt;
}

// Local tile -> (m-tile, n-tile): bands of BAND m-tiles; inside a band the
// m-tiles of one n-tile are adjacent, then the next n-tile.
template <int BAND = GM_BAND>
__device__ __forceinline__ void gm_band(int local, int mtiles, int nt, int* m, int* n)
{
    const int full = mtiles / BAND;
    if (local < full * BAND * nt) {
        const int band = local / (BAND * nt), rem = local % (BAND * nt);
        *n = rem / BAND;
        *m = band * BAND + rem % BAND;
    } else {
        const int rem = local - full * BAND * nt, bm = mtiles - full * BAND;
        *n = rem / bm;
        *m = full * BAND + rem % bm;
    }
}

// Global weight row of tile row i, or -1 past the output width.  gate/up:
// 32-row block b = i/32 holds gate (b%4 < 2) or up rows of output columns
// 64*(b/4) + 32*(b%2) + i%32 of the tile.
template <bool GATE_UP>
__device__ __forceinline__ long long gm_wrow(const FfnArgs& a, int e, int n0, int NOUT, int i)
{
    if constexpr (GATE_UP) {
        const int b = i >> 5;
        const int n = n0 + 64 * (b >> 2) + 32 * (b & 1) + (i & 31);
        if (n >= NOUT) return -1;
        return (long long)e * 2 * a.I + ((b & 2) ? a.I + n : n);
    } else {
        const int n = n0 + i;
        return n < NOUT ? (long long)e * a.H + n : -1;
    }
}


}  // namespace moe
