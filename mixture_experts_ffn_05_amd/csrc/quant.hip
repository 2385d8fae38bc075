// MXFP4 quantiser and fake quantiser: the step that turns bf16 expert
// weights into the MXFP4 bytes the layer consumes, and its
// quantise-then-decode form, which training through quantisation uses in the
// forward pass ("Persona Kappa: training a 20B LLM on desktop GPUs", section
// "Quantization-Aware Training (QAT)": fake-quantised expert weights during
// QAT, then the MXFP4 export).
//
// Rule (OCP Microscaling v1.0; the pages do not print one): per block of 32
// consecutive elements along a row, with amax = max |v|,
//   X = floor(log2 amax) - 2,  S = clamp(X + 127, 0, 254)   (E8M0 byte),
//   an all-zero block stores S = 0;
//   each element v / 2^(S-127) is rounded to the nearest E2M1 value with ties
//   to the even code (|v| / 2^(S-127) < 8 always, since amax < 2^(X+3)), and
//   a zero result carries no sign bit.
//
// The tensor is a flat run of 32-element blocks: element offset 32g is block
// g, whose packed bytes sit at 16g and whose scale byte at g, whatever the
// row length.  Four lanes share a block, eight elements (one 16-byte load)
// each: a wave reads 1 KB of consecutive input and writes 256 consecutive
// packed bytes.  The block's amax meets across the four lanes by two DPP
// quad permutes.  The elements are rounded by v_cvt_scalef32_pk_fp4_bf16,
// which divides by the scale's power of two and rounds to nearest even on the
// E2M1 grid; the negative-zero codes it leaves are cleared afterwards.
//
// HBM-bound: 2 B read + 17/32 B written per element (quantise), 2 + 2 B
// (fake quantise).
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// Launch shape (measured on the 20b gate/up tensor): 128-thread workgroups;
// each thread issues its 16-byte loads for all its slots first, two slots
// when quantising, one when fake quantising (whose output is 4x larger).
constexpr int Q_THREADS = 128;
template <bool FAKE>
constexpr int q_unroll() { return FAKE ? 1 : 2; }

using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));

// Largest of the four lanes' values in this lane's quad.
__device__ __forceinline__ uint32_t quad_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // lanes ^1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // lanes ^2
    return v;
}

// E8M0 scale byte of a block from the bit pattern of its largest |v| (a
// positive bf16 pattern, 0 for an all-zero block).
__device__ __forceinline__ uint32_t block_scale_byte(uint32_t amax)
{
    if (amax == 0) return 0;
    const int e8 = (int)(amax >> 7);
    // floor(log2 amax): normal bf16 from the exponent field; a subnormal is
    // m * 2^-133 with m the 7-bit mantissa
    const int fl = e8 > 0 ? e8 - 127 : (31 - __builtin_clz(amax & 0x7Fu)) - 133;
    const int s = fl - 2 + 127;
    return (uint32_t)(s < 0 ? 0 : (s > 254 ? 254 : s));
}

// The float 2^(S-127) as the conversion instructions take it (S = 0 gives the
// subnormal 2^-127).
__device__ __forceinline__ float scale_float(uint32_t S)
{
    return S == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(S << 23);
}

// The two codes of one bf16 pair as a byte, element 0 in bits 3:0.  Only the
// byte-0 form of the conversion is used: its element order was checked
// against the rule for every bf16 input and scale; the other byte positions
// place the pair's nibbles the other way round.
__device__ __forceinline__ uint32_t quantize2(uint32_t pair, float sc)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, pair), sc, 0) & 0xFFu;
}

// Codes of 8 elements (two per bf16 pair of v) as 8 nibbles, element 0 in
// bits 3:0.  A nibble whose magnitude is zero loses its sign bit.
__device__ __forceinline__ uint32_t quantize8(u32x4 v, float sc)
{
    const uint32_t c = quantize2(v.x, sc) | (quantize2(v.y, sc) << 8) | (quantize2(v.z, sc) << 16) |
                       (quantize2(v.w, sc) << 24);
    const uint32_t nz = (c | (c >> 1) | (c >> 2)) & 0x11111111u;  // bit 0 of each nibble: magnitude != 0
    return c & (0x77777777u | (nz << 3));
}

// Largest |v| bit pattern of 8 bf16 values (|v| orders as its bits do).
__device__ __forceinline__ uint32_t amax8(u32x4 v)
{
    using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
    auto mag = [](uint32_t p) { return __builtin_bit_cast(u16x2, p & 0x7FFF7FFFu); };
    const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(mag(v.x), mag(v.y)),
                                              __builtin_elementwise_max(mag(v.z), mag(v.w)));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// FAKE = false: packed [N/2] bytes + scales [N/32]; FAKE = true: bf16 [N] of
// the decoded values.  N = 8 * n_slots elements.
template <bool FAKE>
__global__ __launch_bounds__(Q_THREADS) void mxfp4_quant_kernel(const uint16_t* __restrict__ w, int64_t n_slots,
                                                               uint32_t* __restrict__ packed,
                                                               uint8_t* __restrict__ scales,
                                                               uint16_t* __restrict__ out)
{
    constexpr int Q_UNROLL = q_unroll<FAKE>();
    const int64_t base = (int64_t)blockIdx.x * (Q_THREADS * Q_UNROLL) + threadIdx.x;
    u32x4 v[Q_UNROLL];
#pragma unroll
    for (int u = 0; u < Q_UNROLL; ++u) {
        const int64_t slot = base + (int64_t)u * Q_THREADS;
        // slot counts are multiples of 4 and a quad's slots are consecutive
        // from a multiple of 4, so a quad is all in range or all out
        v[u] = slot < n_slots ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w) + slot)
                              : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < Q_UNROLL; ++u) {
        const int64_t slot = base + (int64_t)u * Q_THREADS;
        if (slot >= n_slots) continue;
        const uint32_t S = block_scale_byte(quad_max(amax8(v[u])));
        const float sc = scale_float(S);
        const uint32_t codes = quantize8(v[u], sc);
        if constexpr (!FAKE) {
            __builtin_nontemporal_store(codes, packed + slot);  // streamed out, not re-read here
            if ((threadIdx.x & 3) == 0) scales[slot >> 2] = (uint8_t)S;
        } else {
            u32x4 d;
            d.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
            d.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
            d.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
            d.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
            __builtin_nontemporal_store(d, reinterpret_cast<u32x4*>(out) + slot);
        }
    }
}

static hipError_t launch_quant(bool fake, const uint16_t* w, int64_t n_elems, uint8_t* packed, uint8_t* scales,
                               uint16_t* out, hipStream_t s)
{
    const int64_t n_slots = n_elems / 8;
    const int64_t per_block = Q_THREADS * (fake ? q_unroll<true>() : q_unroll<false>());
    const int64_t grid = (n_slots + per_block - 1) / per_block;
    if (fake)
        hipLaunchKernelGGL(mxfp4_quant_kernel<true>, dim3((unsigned)grid), dim3(Q_THREADS), 0, s, w, n_slots, nullptr,
                           nullptr, out);
    else
        hipLaunchKernelGGL(mxfp4_quant_kernel<false>, dim3((unsigned)grid), dim3(Q_THREADS), 0, s, w, n_slots,
                           reinterpret_cast<uint32_t*>(packed), scales, nullptr);
    return hipGetLastError();
}

// Largest tensor one launch covers (grid x-dimension below 2^31 at the
// smallest slots-per-workgroup).
int64_t mxfp4_quant_max_elems() { return (int64_t)0x7FFFFFFF * Q_THREADS * 8; }

hipError_t launch_mxfp4_quantize(const uint16_t* w, int64_t n_elems, uint8_t* packed, uint8_t* scales, hipStream_t s)
{
    return launch_quant(false, w, n_elems, packed, scales, nullptr, s);
}

hipError_t launch_mxfp4_fakequant(const uint16_t* w, int64_t n_elems, uint16_t* out, hipStream_t s)
{
    return launch_quant(true, w, n_elems, nullptr, nullptr, out, s);
}

// ---------------------------------------------------------------------------
// Packed MXFP4 order.  A one-time reordering of an MXFP4 expert tensor for the
// decode-regime kernel (it moves bytes and changes no value; the order is
// documented with moe_mxfp4_pack).  One thread per 16-byte piece (one row over
// one 32-element K-block): the read side walks the row-major tensor in order,
// the piece and its scale byte are written to their packed positions.
__global__ __launch_bounds__(256) void mxfp4_pack_kernel(int gate_up, int I, int R, int nkb, long long n_pieces,
                                                        const u32x4* __restrict__ w, const uint8_t* __restrict__ s,
                                                        uint8_t* __restrict__ wp, uint8_t* __restrict__ sp)
{
    const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    if (id >= n_pieces) return;
    const int kb = (int)(id % nkb);
    const long long er = id / nkb;  // expert * R + row
    const long long e = er / R;
    const int r = (int)(er % R);
    int it, q;
    if (gate_up) {  // item it: gate columns 16it..16it+15 in slots 0-15, the matching up rows in 16-31
        const int n = r < I ? r : r - I;
        it = n / 16;
        q = n % 16 + (r < I ? 0 : 16);
    } else {        // item it: rows 32it..32it+31
        it = r / 32;
        q = r % 32;
    }
    const int g = q >> 2, t = q & 3, c = kb >> 4, b = kb & 15;
    const int nb = min(16, nkb - 16 * c);
    const long long wo = e * R * (long long)nkb * 16 + (long long)it * 512 * nkb + 8192ll * c + 64 * g * nb +
                         16 * (4 * b + t);
    const long long so = e * R * (long long)nkb + (long long)it * 32 * nkb + 512ll * c + 8 * (4 * b + t) + g;
    *reinterpret_cast<u32x4*>(wp + wo) = w[id];
    sp[so] = s[id];
}

hipError_t launch_mxfp4_pack(bool gate_up, int E, int I, int H, const uint8_t* w, const uint8_t* s, uint8_t* wp,
                             uint8_t* sp, hipStream_t st)
{
    const int R = gate_up ? 2 * I : H, K = gate_up ? H : I;
    const long long n = (long long)E * R * (K / 32);
    const long long grid = (n + 255) / 256;
    hipLaunchKernelGGL(mxfp4_pack_kernel, dim3((unsigned)grid), dim3(256), 0, st, gate_up ? 1 : 0, I, R, K / 32, n,
                       reinterpret_cast<const u32x4*>(w), s, wp, sp);
    return hipGetLastError();
}

}  // namespace moe
