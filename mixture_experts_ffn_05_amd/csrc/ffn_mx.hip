// MXFP4 grouped expert GEMM on the CDNA4 MX matrix cores (prefill regime).
//
// The expert weights are natively MXFP4 while the activations stay bf16
// (Persona Kappa post, section "Quantization-Aware Training (QAT)": W4A16).
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies block-scaled operands -- here
// E2M1 weights by E2M3 (FP6) activations, one E8M0 scale per 32 K-values of
// each operand -- at four times the multiply-accumulates per instruction of
// the bf16 32x32x16 MFMA for the same issue time.  One E2M3 term is too coarse
// for bf16 activations (3 mantissa bits, one exponent per 32 values), so each
// activation block is split in two terms before the GEMM:
//   hi = x rounded to the E2M3 grid with the block's OCP scale
//        2^(floor(log2 amax) - 2)  (round to nearest even, saturating),
//   lo = (x - hi) rounded the same way with its own block scale,
// and every product is the sum of two MFMAs, W*hi + W*lo.  hi has 4
// significant bits and lo carries the next 4, so hi + lo keeps about as much
// of x as bf16 does while both MFMAs together still take half the issue time
// of the bf16 product.  The weight codes and scales go to the matrix cores as
// stored, with no decode.
//
// mx_split_kernel makes the two terms once per activation row (x before the
// gate/up GEMM, and h before the down GEMM where h arrives as bf16; the layer
// entry points have the gate/up epilogue split h itself).  mx_gemm_kernel is
// the grouped GEMM, with the tile schedule and gate/up pairing of the bf16
// tiled kernel (tile_sched.h):
//   tile 256 weight rows x 256 tokens, 8 waves (two per SIMD) as 2 weight
//   halves x 4 token quarters, each wave 4 x 2 blocks of 32 x 32 in 128
//   accumulators; K advances in stages of 64 (two MX blocks: one MFMA per
//   block pair and term) through a ring of 4 LDS buffers.  With two waves per
//   SIMD one wave's MFMAs run while the other waits on LDS or at a barrier.
// Token codes and scales go straight into LDS (buffer loads to LDS) three
// stages ahead.  Each tile row stays whole in LDS (its six 16-byte chunks of a stage
// in rotated slots, see mx_chunk_slot), so one wave-wide load reads
// consecutive 16-byte pieces of gathered rows and the fragment reads are free
// of bank conflicts.  Weight codes and scales take registers two stages ahead
// (so that the row-major and packed MXFP4 orders are addressed alike) and are
// stored to LDS as [block][row][16 B].
#include <string.h>

#include <type_traits>

#include "moe_device.h"
#include "moe_kernels.h"
#include "tile_sched.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(32))) __bf16 bf16x32;
typedef __attribute__((ext_vector_type(6))) unsigned int u32x6;
typedef __attribute__((ext_vector_type(8))) unsigned int u32x8;
typedef __attribute__((ext_vector_type(12))) unsigned int u32x12;

// ------------------------------------------------------------------ split

constexpr int MXS_THREADS = 256;
constexpr int MX_CODE_BYTES = 48;  // per 32-element block: hi codes (24 B), then lo codes (24 B)

// OCP shared exponent of a block as its E8M0 byte: floor(log2 amax) - 2 (2 =
// the largest E2M3 exponent), from the fp32/bf16 exponent field of amax;
// clamped to [1, 254] so that the scale 2^(S-127) is a normal float (blocks
// that small round to zero either way).
__device__ __forceinline__ int mx_shared_exponent(uint32_t amax_exp_field)
{
    return min(max((int)amax_exp_field - 2, 1), 254);
}

// Both terms of one 32-element block, w = its bf16 values in order, two per
// dword (element 2i in the low half of w[i]).  hi's codes come from the
// hardware conversion (round to nearest even of x / 2^(S-127) onto E2M3,
// saturating at 7.5); hi's values are formed the same way in fp32 to get
// lo = x - hi, which is exact and exactly a bf16 value (x and hi are both
// multiples of x's last bit, and |lo| <= |x|).  Writes the 48 code bytes as
// three 16-byte pieces and returns the two scale bytes (hi in the low byte).
__device__ __forceinline__ uint32_t mx_split_block(const uint32_t (&w)[16], u32x4 (&out)[3])
{
    uint32_t amax = 0;  // largest |x| as bf16 bits
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    const int S = mx_shared_exponent(amax >> 7);
    const float inv = __uint_as_float((uint32_t)(254 - S) << 23);  // 2^(127 - S)
    const float sc = __uint_as_float((uint32_t)S << 23);           // 2^(S - 127)
    float lo[32];
    float lmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float f = (j & 1) ? bf16_hi(w[j / 2]) : bf16_lo(w[j / 2]);
        const float v = f * inv;  // exact (power-of-two scaling)
        // round to a multiple of the E2M3 step at |v|: 2^(max(floor(log2|v|), 0) - 3),
        // by adding and subtracting 1.5 * 2^(23 + log2 step) (nearest even)
        const int e = max((int)((__float_as_uint(v) >> 23) & 0xFFu) - 127, 0);
        const float big = __uint_as_float(((uint32_t)(e + 147) << 23) | 0x00400000u);
        float r = __fsub_rn(__fadd_rn(v, big), big);
        r = fminf(fmaxf(r, -7.5f), 7.5f);
        lo[j] = __fsub_rn(f, __fmul_rn(r, sc));
        lmax = fmaxf(lmax, fabsf(lo[j]));
    }
    const int S2 = mx_shared_exponent(__float_as_uint(lmax) >> 23);
    const float sc2 = __uint_as_float((uint32_t)S2 << 23);
    uint32_t lw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        lw[i] = (__float_as_uint(lo[2 * i]) >> 16) | (__float_as_uint(lo[2 * i + 1]) & 0xFFFF0000u);
    const u32x6 ch = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32, w), sc);
    const u32x6 cl = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(__builtin_bit_cast(bf16x32, lw), sc2);
    out[0] = u32x4{ch[0], ch[1], ch[2], ch[3]};
    out[1] = u32x4{ch[4], ch[5], cl[0], cl[1]};
    out[2] = u32x4{cl[2], cl[3], cl[4], cl[5]};
    return (uint32_t)S | ((uint32_t)S2 << 8);
}

// One lane per 32-element block.
__global__ __launch_bounds__(MXS_THREADS) void mx_split_kernel(const uint16_t* __restrict__ in, int64_t nblocks,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales)
{
    const int64_t blk = (int64_t)blockIdx.x * MXS_THREADS + threadIdx.x;
    if (blk >= nblocks) return;
    const u32x4* src = reinterpret_cast<const u32x4*>(in + blk * 32);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
    u32x4 c[3];
    const uint32_t sb = mx_split_block(w, c);
    u32x4* dst = reinterpret_cast<u32x4*>(codes + blk * MX_CODE_BYTES);
    dst[0] = c[0];
    dst[1] = c[1];
    dst[2] = c[2];
    *reinterpret_cast<uint16_t*>(scales + blk * 2) = (uint16_t)sb;
}

hipError_t launch_mx_split(const uint16_t* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s)
{
    const int64_t nblocks = rows * (K / 32);
    if (nblocks == 0) return hipSuccess;
    const int64_t grid = (nblocks + MXS_THREADS - 1) / MXS_THREADS;
    hipLaunchKernelGGL(mx_split_kernel, dim3((unsigned)grid), dim3(MXS_THREADS), 0, s, in, nblocks, codes, scales);
    return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM

constexpr int MX_THREADS = 512;
constexpr int MX_WAVES = MX_THREADS / WAVE;  // 8: 2 weight halves x 4 token quarters, two per SIMD
constexpr int MX_NBUF = 4;                   // LDS stages
constexpr int MX_DIST = 3;                   // token loads run this many stages ahead
constexpr int MX_WB = 4;                     // weight blocks per wave (128 rows)
constexpr int MX_TB = 2;                     // token blocks per wave (64 tokens)
constexpr int MX_BAND = 4;                   // M-tiles per band of the tile order
constexpr int MX_XCH = 2 * MX_CODE_BYTES / 16;  // 16-byte token code chunks per row and stage (6)
constexpr int MX_XL = MX_XCH * GM_BT * 16 / 1024 / MX_WAVES;  // token code loads per wave per stage (3)
constexpr int MX_SW = GM_BT / WAVE;  // waves that load token scales, 64 rows x 4 B each (4)

struct MxShared {
    uint8_t w[MX_NBUF][2][GM_BW][16];          // E2M1 codes: [block][row], 32 values per 16 B
    uint8_t ws[MX_NBUF][2][GM_BW];             // weight E8M0 scales [block][row]
    uint8_t x[MX_NBUF][GM_BT][MX_XCH][16];     // token codes [row][chunk slot], see mx_chunk_slot
    uint8_t xs[MX_NBUF][GM_BT][2][2];          // token scales [row][block][hi, lo]
};

// Token code chunk j (0..5: chunks 0-2 of block 0, then of block 1) of tile
// row r sits in slot (j - ((r / 8) % 2)) mod 6 of the row's 96 LDS bytes: the
// 16 lanes of one LDS read pass (16 consecutive rows, one chunk) then cover
// 16 distinct 4-bank groups, and the rows stay whole in LDS so that each
// wave-wide global load reads whole row segments.
__device__ __forceinline__ int mx_chunk_slot(int r, int j) { return (j + 6 - ((r >> 3) & 1)) % 6; }

// One 32x32x64 block-scaled MFMA: E2M1 weights (format 4) by one E2M3 term
// (format 2) of the tokens; the weight scale is byte 0 of wsc, the token
// term's scale byte TERM of xsc (0: hi, 1: lo).
template <int TERM>
__device__ __forceinline__ f32x16 mfma_mx(u32x4 w, u32x6 x, uint32_t wsc, uint32_t xsc, f32x16 c)
{
    const i32x8 a = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    const i32x8 b = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)x[4], (int)x[5], 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 2, 0, (int)wsc, TERM, (int)xsc);
}

template <bool PACKED, bool GATE_UP, bool SPLIT_OUT>
__global__ __launch_bounds__(MX_THREADS, 1) void mx_gemm_kernel(FfnArgs a)
{
    __shared__ __attribute__((aligned(16))) MxShared sh;
    const int NOUT = GATE_UP ? a.I : a.H;  // output columns
    const int K = GATE_UP ? a.H : a.I;
    const int nkb = K / 32;
    const int nstages = K / 64;
    const int WCOLS = GATE_UP ? GM_BW / 2 : GM_BW;  // output columns per tile
    const int nt = (NOUT + WCOLS - 1) / WCOLS;

    // ---- tile of this block (the bf16 tiled kernel's schedule)
    const int total = gm_total_tiles(a.offsets, a.E, nt);
    const int per = (total + 7) / 8;
    if ((int)blockIdx.x / 8 >= per) return;  // uniform per block
    const int tile = (blockIdx.x % 8) * per + blockIdx.x / 8;
    if (tile >= total) return;
    int local, mtiles, mt, ntile;
    const int e = gm_locate(a.offsets, a.E, nt, tile, &local, &mtiles);
    gm_band<MX_BAND>(local, mtiles, nt, &mt, &ntile);
    const int seg1 = a.offsets[e + 1], sbase = a.offsets[e] + mt * GM_BT;
    const int n0 = ntile * WCOLS;

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int r32 = lane & 31, kg = lane >> 5;
    // Weight half and token quarter of this wave.  Waves w and w + 4 share a
    // SIMD and take token quarters two apart, so that in an expert's last,
    // partly filled tile every SIMD keeps a wave with tokens: a wave whose
    // quarter lies wholly past the segment skips its fragment reads and MFMAs
    // (it still stages its share of the loads and meets every barrier).
    const int ww = wave / 4, wt = (wave + 2 * ww) % 4;
    const bool live = sbase + 32 * MX_TB * wt < seg1;

    // Activation row of tile row `row` (rows past the segment read a valid row;
    // their results are never stored).
    auto act_row = [&](int row) -> uint32_t {
        const int s = sbase + row;
        if constexpr (GATE_UP)
            return (uint32_t)(s < seg1 ? a.sorted_pairs[s] / a.k : 0);
        else
            return (uint32_t)(s < seg1 ? s : 0);
    };
    // ---- token codes and scales, straight into LDS by buffer loads whose
    // 32-bit lane offsets stay fixed for the tile (the stage's offset is a
    // scalar).  Codes: the tile's 256 rows x 6 chunk slots are filled in order,
    // 1 KB (64 slots) per wave-wide load; load i of wave w covers slots
    // 64 (w + 8 i) .. +63, and the lane of slot s fetches the chunk that
    // belongs there: row s / 6, chunk j with mx_chunk_slot(row, j) = s % 6.
    // Consecutive lanes so read consecutive 16-byte pieces of the same gathered
    // row.  Scales: waves 0-3, wave w filling rows 64 w .. +63, lane l the 4
    // bytes (hi, lo of both blocks of the stage) of row 64 w + l.  Byte offsets
    // stay below 2^31 (the split arrays of one call are checked against that
    // on the host).
    uint32_t xoff[MX_XL];
#pragma unroll
    for (int i = 0; i < MX_XL; ++i) {
        const int slot = 64 * (wave + MX_WAVES * i) + lane, row = slot / MX_XCH, pos = slot % MX_XCH;
        const int j = (pos + ((row >> 3) & 1)) % MX_XCH;  // inverse of mx_chunk_slot
        xoff[i] = act_row(row) * (uint32_t)(nkb * MX_CODE_BYTES) + j * 16;
    }
    const uint32_t soff = act_row(WAVE * (wave % MX_SW) + lane) * (uint32_t)(nkb * 2);
    const int arows = GATE_UP ? a.T : a.T * a.k;  // rows of the split activations
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.a_codes), (short)0, arows * nkb * MX_CODE_BYTES, 0x00020000);
    const __amdgpu_buffer_rsrc_t xsrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.a_scales), (short)0, arows * nkb * 2, 0x00020000);

    typedef __attribute__((address_space(3))) void* lptr_t;
    auto issue = [&](int st) {
        const int buf = st % MX_NBUF, kk = min(st, nstages - 1);
#pragma unroll
        for (int i = 0; i < MX_XL; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lptr_t)(&sh.x[buf][0][0][0] + 1024 * (wave + MX_WAVES * i)), 16,
                                                     xoff[i], kk * 2 * MX_CODE_BYTES, 0, 0);
        if (wave < MX_SW)  // uniform per wave
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrs, (lptr_t)&sh.xs[buf][WAVE * wave][0][0], 4, soff, kk * 4, 0, 0);
    };

    // ---- weight codes and scales through registers: thread t takes the
    // 16-byte piece (32 codes) of tile row t % 256 at K-block 2 st + t / 256
    // and its scale byte.  Rows past the output width read the tile's first
    // row.  Offsets are 32-bit inside expert e's weights and scales (the host
    // checks that one expert's weights stay below 2^31 bytes).
    const int wr_ = tid % GM_BW, wb2 = tid / GM_BW;  // this thread's weight row and K-block of a stage
    const int R = GATE_UP ? 2 * a.I : a.H;  // weight rows per expert
    long long qrow = gm_wrow<GATE_UP>(a, e, n0, NOUT, wr_);
    if (qrow < 0) qrow = gm_wrow<GATE_UP>(a, e, 0, NOUT, 0);
    const int r = (int)(qrow - (long long)e * R);  // row inside the expert
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.w) + (size_t)e * R * (K / 2)), (short)0, R * (K / 2),
        0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.w_scale + (size_t)e * R * nkb), (short)0, R * nkb, 0x00020000);
    // Packed MXFP4 order (moe_mxfp4_pack): the piece of K-block kb = 16c + b and
    // its scale sit at wo + 8192c + 64 g nb(c) + 64b and so + 512c + 32b, with
    // slot 4g + t of item `it` fixed per thread.  Row-major: wo + 16 kb, so + kb.
    uint32_t wo, so;
    int pg = 0;
    if constexpr (PACKED) {
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
        wo = (uint32_t)it * 512u * nkb + 16u * (q % 4);
        so = (uint32_t)it * 32u * nkb + 8u * (q % 4) + pg;
    } else {
        wo = (uint32_t)r * (uint32_t)(K / 2);
        so = (uint32_t)r * (uint32_t)nkb;
    }
    u32x4 wq[2];
    uint32_t wsc[2];
    auto fetch_w = [&](int set, int st) {
        const int kb = 2 * min(st, nstages - 1) + wb2;
        uint32_t off, soff;
        if constexpr (PACKED) {
            const int c = kb >> 4, b = kb & 15, nb = min(16, nkb - 16 * c);
            off = wo + 8192u * c + 64u * pg * nb + 64u * b;
            soff = so + 512u * c + 32u * b;
        } else {
            off = wo + 16u * kb;
            soff = so + kb;
        }
        wq[set] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
        wsc[set] = __builtin_amdgcn_raw_buffer_load_b8(srs, soff, 0, 0);
    };
    auto store_w = [&](int set, int buf) {
        *reinterpret_cast<u32x4*>(&sh.w[buf][wb2][wr_][0]) = wq[set];
        sh.ws[buf][wb2][wr_] = (uint8_t)wsc[set];
    };
    // vector-memory operations per wave per stage: token loads (codes, and
    // scales in waves 0-3), weight register loads
    constexpr int L = MX_XL + 1, QL = 2;

    f32x16 acc[MX_WB][MX_TB];
#pragma unroll
    for (int m = 0; m < MX_WB; ++m)
#pragma unroll
        for (int t = 0; t < MX_TB; ++t) acc[m][t] = f32x16{};

    // Operand fragments: lane l multiplies K-block kg = l / 32 of weight row
    // 128 ww + 32 m + l % 32 and token row 64 wt + 32 t + l % 32.  A token
    // block's 48 code bytes sit in LDS as three 16-byte chunks c0 | c1 | c2
    // (hi = c0 + the first half of c1, lo = the second half of c1 + c2) and
    // are read into 12 consecutive registers: the hi operand is the first 6,
    // the lo operand the last 6.  Every fragment set has one copy, refilled
    // after its last use in the lo MFMAs: a token block's codes once its four
    // lo MFMAs are issued, the weights during the last token block's.
    u32x4 fw[MX_WB];
    uint32_t fws[MX_WB], fxs[MX_TB];
    u32x12 fx[MX_TB];
    auto chunk = [&](int buf, int c, int t) {
        const int row = 32 * MX_TB * wt + 32 * t + r32;
        return *reinterpret_cast<const u32x4*>(&sh.x[buf][row][mx_chunk_slot(row, 3 * kg + c)][0]);
    };
    auto load_w = [&](int buf, int m) {
        const int row = 128 * ww + 32 * m + r32;
        fw[m] = *reinterpret_cast<const u32x4*>(&sh.w[buf][kg][row][0]);
        fws[m] = sh.ws[buf][kg][row];
    };
    auto load_hi = [&](int buf, int t) {
        const u32x4 c0 = chunk(buf, 0, t), c1 = chunk(buf, 1, t), c2 = chunk(buf, 2, t);
        fx[t] = u32x12{c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w, c2.x, c2.y, c2.z, c2.w};
        fxs[t] = *reinterpret_cast<const uint16_t*>(&sh.xs[buf][32 * MX_TB * wt + 32 * t + r32][kg][0]);
    };
    auto first6 = [](const u32x12& v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5); };
    auto last6 = [](const u32x12& v) { return __builtin_shufflevector(v, v, 6, 7, 8, 9, 10, 11); };
    // hi-term MFMAs of stage `buf`
    auto phase_hi = [&](int buf) {
#pragma unroll
        for (int t = 0; t < MX_TB; ++t) {
#pragma unroll
            for (int m = 0; m < MX_WB; ++m)
                acc[m][t] = mfma_mx<0>(fw[m], first6(fx[t]), fws[m], fxs[t], acc[m][t]);
        }
    };
    // lo-term MFMAs, token block by token block, with the reads of stage `nb`'s
    // fragments as their registers free up
    auto phase_lo = [&](int nb) {
        uint32_t xs_now[MX_TB];
#pragma unroll
        for (int t = 0; t < MX_TB; ++t) xs_now[t] = fxs[t];
#pragma unroll
        for (int t = 0; t < MX_TB; ++t) {
#pragma unroll
            for (int m = 0; m < MX_WB; ++m) {
                acc[m][t] = mfma_mx<1>(fw[m], last6(fx[t]), fws[m], xs_now[t], acc[m][t]);
                if (t == MX_TB - 1) load_w(nb, m);
            }
            load_hi(nb, t);
        }
    };

    // Software pipeline, one K stage (64) per step.  Its 8 hi-term MFMAs are
    // issued first and keep the matrix pipe busy while the wave stores the
    // next stage's weights, issues the weight loads of stage st+3 and waits
    // at the barrier that publishes stage st+1; its 8 lo-term MFMAs then run
    // while stage st+1's fragments are read.  Token loads run MX_DIST stages
    // ahead, weight register loads two.  Every stage runs the same code: the
    // last one's reads of a next stage find the surplus loads (a re-read of
    // the last stage) and are unused.
    for (int st = 0; st < MX_DIST; ++st) issue(st);
    fetch_w(0, 0);
    fetch_w(1, 1);
    store_w(0, 0);
    fetch_w(0, 2);
    vm_wait<0>();
    lds_barrier();
    if (live) {
#pragma unroll
        for (int m = 0; m < MX_WB; ++m) load_w(0, m);
#pragma unroll
        for (int t = 0; t < MX_TB; ++t) load_hi(0, t);
    }
    auto stage = [&](int st, auto set_c) {
        constexpr int SET = decltype(set_c)::value;
        const int buf = st % MX_NBUF, nb = (st + 1) % MX_NBUF;
        __builtin_amdgcn_sched_barrier(0);
        if (live) phase_hi(buf);
        store_w(SET, nb);  // stage st+1, fetched two stages ago
        fetch_w(SET, st + 3);
        // outstanding after this wave's token loads of stage st+1: weight loads
        // of st+2, token loads of st+2, weight loads of st+3
        if (wave < MX_SW)
            vm_wait<L + 2 * QL>();
        else
            vm_wait<L - 1 + 2 * QL>();
        lds_barrier();  // stage st+1 visible; the buffer of stage st-1 is free
        issue(st + MX_DIST);
        __builtin_amdgcn_sched_barrier(0);
        if (live) phase_lo(nb);
    };
    int st = 0;
    for (; st + 1 < nstages; st += 2) {
        stage(st, std::integral_constant<int, 1>{});
        stage(st + 1, std::integral_constant<int, 0>{});
    }
    if (st < nstages) stage(st, std::integral_constant<int, 1>{});
    mfma_drain();
    vm_wait<0>();  // the surplus loads past the last stage

    // ---- epilogue: for each (m, t) the lane holds tile weight rows
    // 128ww + 32m + 8(r/4) + 4(lane/32) + r%4 (r = 0..15) of token
    // 64wt + 32t + lane%32.
    if constexpr (GATE_UP && SPLIT_OUT) {
        // h goes out as the down GEMM's split activations (the bf16 h values
        // split as mx_split_kernel would split them).  Output columns
        // n0 + 64ww + 32m .. +31 (m = 0, 1) are one 32-value block of an h row,
        // held half by lane l (columns 8q + 0..3) and half by lane l ^ 32
        // (8q + 4..7).  The lane pair trades halves so that lane l splits
        // block 0 and lane l ^ 32 block 1 of its token row.
        const int nkb_out = NOUT / 32;
        const int kb = (n0 + 64 * ww) / 32 + kg;
        const bool cols_in = n0 + 64 * ww < NOUT;  // NOUT % 64 == 0: both blocks in or out
#pragma unroll
        for (int t = 0; t < MX_TB; ++t) {
            uint32_t hv[2][8];  // [block m][dword 2q + j]: bf16 pairs of columns 8q + 4kg + 2j, +1
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const f32x16& g = acc[m][t];
                const f32x16& u = acc[m + 2][t];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    hv[m][i] = pack_bf16x2(silu(g[2 * i]) * u[2 * i], silu(g[2 * i + 1]) * u[2 * i + 1]);
            }
            uint32_t mine[8], theirs[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                mine[i] = kg ? hv[1][i] : hv[0][i];
                theirs[i] = (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) * 4, (int)(kg ? hv[0][i] : hv[1][i]));
            }
            uint32_t wv[16];  // the block's 32 values in column order
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wv[4 * q + 0] = kg ? theirs[2 * q] : mine[2 * q];
                wv[4 * q + 1] = kg ? theirs[2 * q + 1] : mine[2 * q + 1];
                wv[4 * q + 2] = kg ? mine[2 * q] : theirs[2 * q];
                wv[4 * q + 3] = kg ? mine[2 * q + 1] : theirs[2 * q + 1];
            }
            u32x4 c[3];
            const uint32_t sb = mx_split_block(wv, c);
            const int s = sbase + 32 * MX_TB * wt + 32 * t + r32;
            if (s < seg1 && cols_in) {
                const size_t blk = (size_t)s * nkb_out + kb;
                u32x4* dst = reinterpret_cast<u32x4*>(a.out_codes + blk * MX_CODE_BYTES);
                dst[0] = c[0];
                dst[1] = c[1];
                dst[2] = c[2];
                *reinterpret_cast<uint16_t*>(a.out_scales + blk * 2) = (uint16_t)sb;
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < MX_TB; ++t) {
        const int s = sbase + 32 * MX_TB * wt + 32 * t + r32;
        if (s >= seg1) continue;
        if constexpr (GATE_UP) {
            // blocks m = 0, 1 are gate columns 64ww + 32m .., blocks m + 2 the matching up
#pragma unroll
            for (int m = 0; m < MX_WB / 2; ++m) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n0 + 64 * ww + 32 * m + 8 * q + 4 * kg;
                    if (col < NOUT) {
                        const f32x16& g = acc[m][t];
                        const f32x16& u = acc[m + MX_WB / 2][t];
                        uint2 o;
                        o.x = pack_bf16x2(silu(g[4 * q + 0]) * u[4 * q + 0], silu(g[4 * q + 1]) * u[4 * q + 1]);
                        o.y = pack_bf16x2(silu(g[4 * q + 2]) * u[4 * q + 2], silu(g[4 * q + 3]) * u[4 * q + 3]);
                        *reinterpret_cast<uint2*>(a.out + (size_t)s * NOUT + col) = o;
                    }
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < MX_WB; ++m) {
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

bool mx_supported(int H, int I)
{
    // K stages of 64; one expert's weights addressed with 32-bit offsets
    return H % 64 == 0 && I % 64 == 0 && (long long)I * H < (1ll << 31);
}

template <bool PACKED, bool GATE_UP, bool SPLIT_OUT>
static hipError_t launch_mx(const FfnArgs& a, hipStream_t s)
{
    const int NOUT = GATE_UP ? a.I : a.H;
    const int WCOLS = GATE_UP ? GM_BW / 2 : GM_BW;
    const long long nt = (NOUT + WCOLS - 1) / WCOLS;
    const long long mt_bound = ((long long)a.T * a.k + GM_BT - 1) / GM_BT + a.E;
    long long grid = nt * mt_bound;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((mx_gemm_kernel<PACKED, GATE_UP, SPLIT_OUT>), dim3((unsigned)grid), dim3(MX_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up_mx(const FfnArgs& a, hipStream_t s)
{
    if (a.out_codes)
        return a.wfmt == 2 ? launch_mx<true, true, true>(a, s) : launch_mx<false, true, true>(a, s);
    return a.wfmt == 2 ? launch_mx<true, true, false>(a, s) : launch_mx<false, true, false>(a, s);
}

hipError_t launch_down_mx(const FfnArgs& a, hipStream_t s)
{
    return a.wfmt == 2 ? launch_mx<true, false, false>(a, s) : launch_mx<false, false, false>(a, s);
}

}  // namespace moe
