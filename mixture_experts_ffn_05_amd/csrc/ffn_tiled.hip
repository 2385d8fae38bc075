// Tiled grouped expert GEMM (prefill regime): many tokens per expert.
//
// Each expert segment of the permutation is an independent GEMM
//   gate/up: [2I weight rows] x [M_e tokens], K = H, token rows gathered from x
//   down:    [H weight rows]  x [M_e rows of h], K = I
// with fp32 accumulation on bf16 MFMA (v_mfma_f32_32x32x16_bf16).  MXFP4
// weights (Persona Kappa post, section "Quantization-Aware Training (QAT)":
// W4A16, activations stay bf16) are decoded to bf16 while being staged into
// LDS.  The gate/up kernel holds gate and up rows of the same output columns
// in one tile and applies silu(gate)*up in registers before writing h.
//
// Tile: 256 weight rows x 256 tokens, 8 waves (two per SIMD, so one wave's
// MFMAs run while the other waits on memory or a barrier) in 2 x 4; a wave
// owns 128 weight rows x 64 tokens = 4 x 2 blocks of 32x32 in 128
// accumulator registers, so per 16-wide K step it reads 6 operand fragments
// from LDS for 8 MFMAs (the next step's fragments are read while the current
// MFMAs run).
// For gate/up the tile's weight rows are ordered [g0 g1 u0 u1 | g2 g3 u2 u3]
// (32-row blocks of gate and up rows of the same 128 output columns), so each
// wave holds matching gate and up blocks.
//
// K advances in stages of 32 (the C-ABI admits only hidden and expert widths
// that are multiples of 32, so there is no K tail) through a ring of 4 LDS
// buffers: bf16 operands
// are loaded straight into LDS with global_load_lds three stages ahead of the
// MFMAs (no staging registers), so each stage's loads have three stages of
// MFMAs to land; MXFP4 weights take a register detour two stages ahead to be
// decoded.  One barrier per stage, placed after the stage's first 16 MFMAs
// are issued so the matrix pipe stays busy through it.  LDS rows are 64 B (32 bf16) with 16-B
// chunks XOR-swizzled by (row/4)%4, so the 16 lanes that read one chunk of 16
// consecutive rows hit 16 distinct bank groups.
//
// Schedule: the grid enumerates tiles in bands of 4 M-tiles per expert, the
// 4 M-tiles of one N-tile adjacent, so neighbouring tiles share token rows or
// weight rows; block b works on tile (b % 8) * ceil(tiles / 8) + b / 8 so that
// the blocks resident on one XCD (dispatched round-robin by block index) take
// a contiguous run of tiles and share its L2.
#include <string.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_kernels.h"
#include "tile_sched.h"

namespace moe {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int GM_THREADS = 512;
constexpr int GM_WAVES = GM_THREADS / WAVE;  // 8: 2 weight halves x 4 token quarters
constexpr int GM_BK = 32;     // K per stage
constexpr int GM_NBUF = 4;    // LDS stages
constexpr int GM_DIST = 3;    // bf16 loads run this many stages ahead
constexpr int GM_WB = 4;      // weight blocks per wave (128 rows)
constexpr int GM_TB = 2;      // token blocks per wave (64 tokens)
constexpr int GM_ROWB = GM_BK * 2;                                   // bytes per LDS row (64)
constexpr int GM_DL = GM_BW * GM_ROWB / 1024 / GM_WAVES;  // direct loads per wave per operand (2)

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Byte offset of 16-B chunk c (0..3) of row r in a [rows][32] bf16 LDS tile.
__device__ __forceinline__ int gm_swz(int r, int c) { return r * GM_ROWB + ((c ^ ((r >> 2) & 3)) << 4); }

struct GmShared {
    uint8_t w[GM_NBUF][GM_BW * GM_ROWB];
    uint8_t x[GM_NBUF][GM_BT * GM_ROWB];
};

// WGRAD (with WFMT = 0, GATE_UP = false): the weight-gradient product of the
// backward, C[e][m][n] = sum_j A_e[m][j] B_e[n][j] over expert e's padded
// segment (Kpad_e a multiple of 64, zero-padded), A_e in the weight role (256
// rows m per tile) and B_e in the token role (256 rows n per tile); tiles
// enumerate (expert, m-tile, n-tile) in the same banded, XCD-grouped order.
template <int WFMT, bool GATE_UP, bool WGRAD>
__global__ __launch_bounds__(GM_THREADS, GM_WAVES / 4) void gemm_kernel(FfnArgs a)
{
    static_assert(!WGRAD || (WFMT == 0 && !GATE_UP), "weight-gradient mode is bf16, no gate/up pairing");
    __shared__ __attribute__((aligned(16))) GmShared sh;
    const int NOUT = WGRAD ? a.wg_M : (GATE_UP ? a.I : a.H);  // output columns (WGRAD: A rows)
    int K = GATE_UP ? a.H : a.I;
    const int WCOLS = GATE_UP ? GM_BW / 2 : GM_BW;  // output columns per tile
    const int nt = (NOUT + WCOLS - 1) / WCOLS;

    // ---- tile of this block
    int total, e, local, mtiles;
    if constexpr (WGRAD) {
        mtiles = (a.wg_N + GM_BT - 1) / GM_BT;  // token-role tiles
        total = a.E * mtiles * nt;
    } else {
        total = gm_total_tiles(a.offsets, a.E, nt);
    }
    [[maybe_unused]] const int tile_w = (int)blockIdx.x;
    if constexpr (WGRAD) {
        // Experts' K differ (their token counts) while each has the same
        // number of tiles, so tiles go out longest first: block b takes tile
        // b % tpe of the expert ranked b / tpe by descending K (ties: lower
        // index first).  Consecutive blocks land on different XCDs, so every
        // expert's tiles spread over the whole chip.
        if (tile_w >= total) return;  // uniform per block
        const int tpe = mtiles * nt;
        const int rank = (int)blockIdx.x / tpe;
        local = (int)blockIdx.x % tpe;
        e = -1;
        for (int base = 0; base < a.E && e < 0; base += WAVE) {
            const int me = base + lane_id();
            const int kme = me < a.E ? a.wg_padoff[me + 1] - a.wg_padoff[me] : -1;
            int r = 0;
            for (int o = 0; o < a.E; ++o) {
                const int ko = a.wg_padoff[o + 1] - a.wg_padoff[o];
                r += (ko > kme || (ko == kme && o < me)) ? 1 : 0;
            }
            const uint64_t hit = ballot(me < a.E && r == rank);
            if (hit) e = base + (int)__builtin_ctzll(hit);
        }
    } else {
        const int per = (total + 7) / 8;
        if ((int)blockIdx.x / 8 >= per) return;  // uniform per block
        const int tile = (blockIdx.x % 8) * per + blockIdx.x / 8;
        if (tile >= total) return;
        e = gm_locate(a.offsets, a.E, nt, tile, &local, &mtiles);
    }
    int mt, ntile;
    gm_band(local, mtiles, nt, &mt, &ntile);
    int seg1 = 0, sbase = 0, p0 = 0;
    if constexpr (WGRAD) {
        p0 = a.wg_padoff[e];
        K = a.wg_padoff[e + 1] - p0;
        sbase = mt * GM_BT;  // first token-role row (a row of B_e)
        seg1 = a.wg_N;
    } else {
        seg1 = a.offsets[e + 1];
        sbase = a.offsets[e] + mt * GM_BT;
    }
    const int n0 = ntile * WCOLS;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int r32 = lane & 31, kg = lane >> 5;
    // Weight half and token quarter of this wave.  Waves w and w + 4 share a
    // SIMD and take token quarters two apart, so that in an expert's last,
    // partly filled tile every SIMD keeps a wave with tokens: a wave whose
    // quarter lies wholly past the segment skips its fragment reads and MFMAs
    // (it still stages its share of the loads and meets every barrier).
    const int ww = wave / 4, wt = (wave + 2 * ww) % 4;
    const bool live = sbase + 32 * GM_TB * wt < seg1;

    // ---- direct-to-LDS staging of bf16 tiles.  Wave w, load i covers tile
    // rows 16(w + 8i) .. +15; lane l lands in LDS slot l of that 1-KB span,
    // i.e. row 16(w + 4i) + l/4, physical chunk l%4, so it fetches logical
    // chunk (l%4) ^ ((row/4)%4) of its row.  Rows past the output width or the
    // segment point at a valid row (their results are never stored).
    const int lrow = lane >> 2, lpc = lane & 3;
    const uint16_t* xsrc[GM_DL];
    const uint16_t* wsrc[GM_DL];
    int lchunk[GM_DL];
#pragma unroll
    for (int i = 0; i < GM_DL; ++i) {
        const int row = 16 * (wave + GM_WAVES * i) + lrow;
        lchunk[i] = lpc ^ ((row >> 2) & 3);
        const int s = sbase + row;
        if constexpr (WGRAD) {
            xsrc[i] = a.wg_b + (size_t)a.wg_N * p0 + (size_t)(s < seg1 ? s : 0) * K;
            const int m = n0 + row;
            wsrc[i] = a.wg_a + (size_t)a.wg_M * p0 + (size_t)(m < NOUT ? m : 0) * K;
            continue;
        }
        if constexpr (GATE_UP)
            xsrc[i] = a.x + (size_t)(s < seg1 ? a.sorted_pairs[s] / a.k : 0) * a.H;
        else
            xsrc[i] = a.a_rows + (size_t)(s < seg1 ? s : 0) * a.I;
        if constexpr (WFMT == 0) {
            const long long wr = gm_wrow<GATE_UP>(a, e, n0, NOUT, row);
            wsrc[i] = static_cast<const uint16_t*>(a.w) + (size_t)(wr >= 0 ? wr : gm_wrow<GATE_UP>(a, e, 0, NOUT, 0)) * K;
        } else {
            wsrc[i] = nullptr;
        }
    }
    typedef __attribute__((address_space(1))) const void* gptr_t;
    typedef __attribute__((address_space(3))) void* lptr_t;
    auto direct = [&](const uint16_t* const (&src)[GM_DL], uint8_t* tile, int kk) {
#pragma unroll
        for (int i = 0; i < GM_DL; ++i) {
            __builtin_amdgcn_global_load_lds((gptr_t)(src[i] + kk + 8 * lchunk[i]), (lptr_t)(tile + 16 * (wave + GM_WAVES * i) * GM_ROWB), 16,
                                             0, 0);
        }
    };

    // ---- MXFP4 weights: thread t stages half qh = t%2 of tile row t/2 (16
    // elements = 8 B, and the row's scale) two stages ahead in registers and
    // decodes it into LDS chunks 2qh, 2qh+1 of the row.  Rows past the output
    // width read the tile's first row (never stored).
    const int nstages = K / GM_BK;
    long long qrow = 0;
    if constexpr (WFMT != 0) {
        qrow = gm_wrow<GATE_UP>(a, e, n0, NOUT, tid >> 1);
        if (qrow < 0) qrow = gm_wrow<GATE_UP>(a, e, 0, NOUT, 0);
    }
    // Packed MXFP4 order (moe_mxfp4_pack): the row's 16-byte piece of K-block
    // kb = 16c + b and its scale sit at pbase + c*8192 + g*64*nb(c) + 64b and
    // psbase + c*512 + 32b, with slot 4g+t of item `it` fixed per thread.
    long long pbase = 0, psbase = 0;
    int pg = 0;
    if constexpr (WFMT == 2) {
        const int R = GATE_UP ? 2 * a.I : a.H, nkb = K / 32;
        const long long eq = qrow / R;
        const int r = (int)(qrow % R);
        int it, q;
        if constexpr (GATE_UP) {
            const int n = r < a.I ? r : r - a.I;
            it = n / 16;
            q = n % 16 + (r < a.I ? 0 : 16);
        } else {
            it = r / 32;
            q = r % 32;
        }
        pg = q / 4;
        pbase = eq * R * (K / 2) + (long long)it * 512 * nkb + 16 * (q % 4);
        psbase = eq * R * nkb + (long long)it * 32 * nkb + 8 * (q % 4) + pg;
    }
    const int qh = tid & 1;
    uint2 qw[2];
    uint8_t qsc[2];  // kept as bytes: widening happens at the decode, not at the load
    // Every load below is issued unconditionally; stages past the end re-read
    // the last stage into a free buffer, so each stage issues the same number
    // of loads and the loop body has no branches.
    auto fetch_q = [&](int set, int st) {
        const int kk = min(st, nstages - 1) * GM_BK;
        if constexpr (WFMT == 2) {
            const int kb = kk / 32, c = kb >> 4, b = kb & 15, nb = min(16, K / 32 - 16 * c);
            const long long off = pbase + 8192ll * c + 64 * pg * nb + 64 * b;
            qw[set] = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.w) + off + 8 * qh);
            qsc[set] = a.w_scale[psbase + 512ll * c + 32 * b];
        } else {
            qw[set] = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(a.w) + qrow * (K / 2) + kk / 2 +
                                                      8 * qh);
            qsc[set] = a.w_scale[qrow * (K / 32) + kk / 32];
        }
    };
    auto store_q = [&](int set, int buf) {
        const float sc = e8m0_to_f32(qsc[set]);
        *reinterpret_cast<u32x4*>(sh.w[buf] + gm_swz(tid >> 1, 2 * qh)) = fp4x8_to_bf16x8(qw[set].x, sc);
        *reinterpret_cast<u32x4*>(sh.w[buf] + gm_swz(tid >> 1, 2 * qh + 1)) = fp4x8_to_bf16x8(qw[set].y, sc);
    };
    // Vector-memory operations per wave per stage (vmcnt bookkeeping): direct
    // loads, and the MXFP4 register loads.
    constexpr int L = (WFMT == 0 ? 2 : 1) * GM_DL;
    constexpr int QL = WFMT != 0 ? 2 : 0;
    // Issue the direct loads of stage st into buffer st % NBUF.
    auto issue = [&](int st) {
        const int buf = st % GM_NBUF, kk = min(st, nstages - 1) * GM_BK;
        if constexpr (WFMT == 0) direct(wsrc, sh.w[buf], kk);
        direct(xsrc, sh.x[buf], kk);
    };

    f32x16 acc[GM_WB][GM_TB];
#pragma unroll
    for (int m = 0; m < GM_WB; ++m)
#pragma unroll
        for (int t = 0; t < GM_TB; ++t) acc[m][t] = f32x16{};

    // Operand fragments of one 16-wide K step, read from LDS.
    struct Frags {
        bf16x8 w[GM_WB];
        bf16x8 x[GM_TB];
    };
    auto load_frags = [&](int buf, int s, Frags& f) {
        const int c = 2 * s + kg;
#pragma unroll
        for (int t = 0; t < GM_TB; ++t)
            f.x[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(sh.x[buf] + gm_swz(32 * GM_TB * wt + 32 * t + r32, c)));
#pragma unroll
        for (int m = 0; m < GM_WB; ++m)
            f.w[m] = as_bf16x8(*reinterpret_cast<const u32x4*>(sh.w[buf] + gm_swz(128 * ww + 32 * m + r32, c)));
    };
    auto mma = [&](const Frags& f) {
#pragma unroll
        for (int m = 0; m < GM_WB; ++m)
#pragma unroll
            for (int t = 0; t < GM_TB; ++t) acc[m][t] = mfma32(f.w[m], f.x[t], acc[m][t]);
    };
    // LDS reads spread evenly among the MFMAs, so their latency hides under them.
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < GM_WB + GM_TB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, GM_WB * GM_TB / (GM_WB + GM_TB), 0);
        }
        if constexpr (GM_WB * GM_TB % (GM_WB + GM_TB) != 0)
            __builtin_amdgcn_sched_group_barrier(0x008, GM_WB * GM_TB % (GM_WB + GM_TB), 0);
    };

    // Software pipeline.  Each stage is two 16-wide K steps.  The barrier that
    // publishes stage st+1 sits between the two halves of stage st: the 16
    // MFMAs of step 0 are issued first and keep the matrix pipe busy while the
    // wave waits at the barrier; step 1's MFMAs then run while stage st+1's
    // first fragments are read.  Direct loads run GM_DIST stages ahead, MXFP4
    // register loads two.  Per stage a wave issues, in order: the register
    // loads of stage st+3, (barrier), the direct loads of stage st+3.
    // (an expert without tokens in the weight-gradient mode has no K: its tile is zero)
    if (!WGRAD || nstages > 0) {
    for (int st = 0; st < GM_DIST; ++st) issue(st);
    if constexpr (WFMT != 0) {
        fetch_q(0, 0);
        fetch_q(1, 1);
        store_q(0, 0);
        fetch_q(0, 2);
    }
    vm_wait<0>();
    lds_barrier();
    Frags f0, f1;
    if (live) load_frags(0, 0, f0);
    // Stage st with st + 1 < nstages.  SET = (st + 1) & 1 is the MXFP4
    // register set holding stage st+1; a template constant, so that the two
    // sets stay in fixed registers.
    auto stage = [&](int st, auto set_c) {
        constexpr int SET = decltype(set_c)::value;
        const int buf = st % GM_NBUF, nb = (st + 1) % GM_NBUF;
        __builtin_amdgcn_sched_barrier(0);
        if (live) {
            load_frags(buf, 1, f1);
            mma(f0);
            interleave();
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (WFMT != 0) {
            store_q(SET, nb);             // stage st+1, fetched two stages ago
            fetch_q(SET, st + 3);
        }
        // Outstanding after this wave's direct loads of stage st+1: register
        // loads of st+2, direct loads of st+2, register loads of st+3.
        vm_wait<L + 2 * QL>();
        lds_barrier();  // stage st+1 visible; buffer of stage st-1 is free
        issue(st + GM_DIST);
        __builtin_amdgcn_sched_barrier(0);
        if (live) {
            load_frags(nb, 0, f0);
            mma(f1);
            interleave();
        }
    };
    int st = 0;
    for (; st + 2 < nstages; st += 2) {
        stage(st, std::integral_constant<int, 1>{});
        stage(st + 1, std::integral_constant<int, 0>{});
    }
    if (st + 1 < nstages) stage(st++, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    if (live) {
        load_frags(st % GM_NBUF, 1, f1);
        mma(f0);
        interleave();
        mma(f1);
    }
    mfma_drain();
    vm_wait<0>();  // the surplus loads past the last stage
    }

    if constexpr (WGRAD) {  // fp32 C[e][m][n]: m = weight-role row, n = token-role row
        float* C = a.wg_out + (size_t)e * a.wg_M * a.wg_N;
#pragma unroll
        for (int t = 0; t < GM_TB; ++t) {
            const int ncol = sbase + 32 * GM_TB * wt + 32 * t + r32;
            if (ncol >= a.wg_N) continue;
#pragma unroll
            for (int m = 0; m < GM_WB; ++m)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int mrow = n0 + 128 * ww + 32 * m + 8 * (r >> 2) + 4 * kg + (r & 3);
                    if (mrow < NOUT) C[(size_t)mrow * a.wg_N + ncol] = acc[m][t][r];
                }
        }
        return;
    }

    // ---- epilogue: for each (m, t) the lane holds tile weight rows
    // 128ww + 32m + 8(r/4) + 4(lane/32) + r%4 (r = 0..15) of token
    // 64wt + 32t + lane%32.
#pragma unroll
    for (int t = 0; t < GM_TB; ++t) {
        const int s = sbase + 32 * GM_TB * wt + 32 * t + r32;
        if (s >= seg1) continue;
        if constexpr (GATE_UP) {
            // blocks m = 0, 1 are gate columns 64ww + 32m .., blocks m + 2 the matching up
#pragma unroll
            for (int m = 0; m < GM_WB / 2; ++m) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n0 + 64 * ww + 32 * m + 8 * q + 4 * kg;
                    if (col < NOUT) {
                        const f32x16& g = acc[m][t];
                        const f32x16& u = acc[m + GM_WB / 2][t];
                        uint2 o;
                        o.x = pack_bf16x2(silu(g[4 * q + 0]) * u[4 * q + 0], silu(g[4 * q + 1]) * u[4 * q + 1]);
                        o.y = pack_bf16x2(silu(g[4 * q + 2]) * u[4 * q + 2], silu(g[4 * q + 3]) * u[4 * q + 3]);
                        *reinterpret_cast<uint2*>(a.out + (size_t)s * NOUT + col) = o;
                        if (a.gu_out) {  // pre-activations kept for the backward
                            uint16_t* gu = a.gu_out + (size_t)s * 2 * NOUT + col;
                            *reinterpret_cast<uint2*>(gu) = uint2{pack_bf16x2(g[4 * q + 0], g[4 * q + 1]),
                                                                  pack_bf16x2(g[4 * q + 2], g[4 * q + 3])};
                            *reinterpret_cast<uint2*>(gu + NOUT) = uint2{pack_bf16x2(u[4 * q + 0], u[4 * q + 1]),
                                                                         pack_bf16x2(u[4 * q + 2], u[4 * q + 3])};
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < GM_WB; ++m) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n0 + 128 * ww + 32 * m + 8 * q + 4 * kg;
                    if (col < NOUT) {
                        const f32x16& v = acc[m][t];
                        uint2 o;
                        o.x = pack_bf16x2(v[4 * q + 0], v[4 * q + 1]);
                        o.y = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
                        *reinterpret_cast<uint2*>(a.out + (size_t)s * NOUT + col) = o;
                    }
                }
            }
        }
    }
}

template <int WFMT, bool GATE_UP>
static hipError_t launch_gemm(const FfnArgs& a, hipStream_t s)
{
    const int NOUT = GATE_UP ? a.I : a.H;
    const int WCOLS = GATE_UP ? GM_BW / 2 : GM_BW;
    const long long nt = (NOUT + WCOLS - 1) / WCOLS;
    const long long mt_bound = ((long long)a.T * a.k + GM_BT - 1) / GM_BT + a.E;
    long long grid = nt * mt_bound;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_kernel<WFMT, GATE_UP, false>), dim3((unsigned)grid), dim3(GM_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up_tiled(const FfnArgs& a, hipStream_t s)
{
    return a.wfmt == 0   ? launch_gemm<0, true>(a, s)
           : a.wfmt == 1 ? launch_gemm<1, true>(a, s)
                         : launch_gemm<2, true>(a, s);
}

hipError_t launch_down_tiled(const FfnArgs& a, hipStream_t s)
{
    return a.wfmt == 0   ? launch_gemm<0, false>(a, s)
           : a.wfmt == 1 ? launch_gemm<1, false>(a, s)
                         : launch_gemm<2, false>(a, s);
}

hipError_t launch_wgrad_tiled(const uint16_t* A, const uint16_t* B, const int32_t* padoff, int E, int M, int N,
                              float* C, hipStream_t s)
{
    FfnArgs a;
    memset(&a, 0, sizeof a);
    a.E = E;
    a.wg_a = A;
    a.wg_b = B;
    a.wg_padoff = padoff;
    a.wg_M = M;
    a.wg_N = N;
    a.wg_out = C;
    const long long grid = (long long)E * ((M + GM_BW - 1) / GM_BW) * ((N + GM_BT - 1) / GM_BT);
    hipLaunchKernelGGL((gemm_kernel<0, false, true>), dim3((unsigned)grid), dim3(GM_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
