// C ABI of the MoE FFN library: argument validation, workspace layout,
// schedule choice and kernel launches.  Declarations and contracts are in
// include/moe.h.  Nothing here allocates, synchronises or copies to the host.
#include <string.h>

#include <string>

#include "moe.h"
#include "moe_kernels.h"

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace regions (byte offsets from the workspace base).  Every entry
// point uses this one layout, so one workspace of moe_workspace_size() bytes
// serves all of them.
struct Layout {
    size_t topk_idx, topk_w, logits, offsets, sorted, rank, perm_scratch, h, y_sorted;
    size_t xs_codes, xs_scales, hs_codes, hs_scales;  // MX path: split x and h (0 bytes when unused)
    size_t total;
};

// The MX path applies: MXFP4 weights, H and I multiples of 64, and split
// activations small enough for the kernel's 32-bit byte offsets.
bool mx_fits(const moe_dims& d)
{
    if (d.wfmt == MOE_WFMT_BF16 || !moe::mx_supported(d.H, d.I)) return false;
    const uint64_t lim = 1ull << 31;
    const uint64_t P = (uint64_t)d.T * (uint64_t)d.k;
    return (uint64_t)d.T * d.H / 32 * 48 < lim && P * d.I / 32 * 48 < lim;
}

Layout layout_for(const moe_dims& d)
{
    const size_t T = (size_t)d.T, P = (size_t)d.T * (size_t)d.k;
    Layout L;
    size_t at = 0;
    auto take = [&](size_t bytes) {
        size_t here = at;
        at = align_up(at + bytes);
        return here;
    };
    L.topk_idx = take(P * sizeof(int32_t));
    L.topk_w = take(P * sizeof(float));
    L.logits = take(T * (size_t)d.E * sizeof(double));
    L.offsets = take(((size_t)d.E + 1) * sizeof(int32_t));
    L.sorted = take(P * sizeof(int32_t));
    L.rank = take(P * sizeof(int32_t));
    L.perm_scratch = take(moe::permute_scratch_bytes((int64_t)P, d.E));
    L.h = take(P * (size_t)d.I * 2);
    L.y_sorted = take(P * (size_t)d.H * 2);
    const bool mx = mx_fits(d);
    L.xs_codes = take(mx ? T * (size_t)d.H / 32 * 48 : 0);
    L.xs_scales = take(mx ? T * (size_t)d.H / 32 * 2 : 0);
    L.hs_codes = take(mx ? P * (size_t)d.I / 32 * 48 : 0);
    L.hs_scales = take(mx ? P * (size_t)d.I / 32 * 2 : 0);
    L.total = at;
    return L;
}

// Sizes within the 32-bit buffer offsets of the packed-order skinny kernel.
bool packed_skinny_fits(const moe_dims& d)
{
    moe::FfnArgs a;
    memset(&a, 0, sizeof a);
    a.T = d.T;
    a.H = d.H;
    a.E = d.E;
    a.k = d.k;
    a.I = d.I;
    return moe::skinny4_supported(a);
}

int check_dims(const moe_dims* d)
{
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->T < 0 || d->H <= 0 || d->E <= 0 || d->k < 1 || d->I <= 0 || d->k > d->E) return MOE_ERR_INVALID_ARG;
    if ((int64_t)d->T * d->k > INT32_MAX) return MOE_ERR_INVALID_ARG;
    if (d->E > 256 || d->k > 8) return MOE_ERR_UNSUPPORTED;
    if (d->H % 32 != 0 || d->I % 32 != 0) return MOE_ERR_UNSUPPORTED;
    if (d->wfmt != MOE_WFMT_BF16 && d->wfmt != MOE_WFMT_MXFP4 && d->wfmt != MOE_WFMT_MXFP4_PACKED)
        return MOE_ERR_UNSUPPORTED;
    if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_TILED_MX) return MOE_ERR_UNSUPPORTED;
    if (d->path == MOE_PATH_TILED_MX && !mx_fits(*d)) return MOE_ERR_UNSUPPORTED;
    if (d->wfmt == MOE_WFMT_MXFP4_PACKED && d->path == MOE_PATH_SKINNY && !packed_skinny_fits(*d))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Null check + alignment check of a device pointer.
int check_ptr(const void* p, size_t a)
{
    if (!p) return MOE_ERR_INVALID_ARG;
    return aligned(p, a) ? MOE_OK : MOE_ERR_MISALIGNED;
}

int check_weights(const moe_dims& d, const moe_expert_weights* w)
{
    if (!w) return MOE_ERR_INVALID_ARG;
    int rc;
    if ((rc = check_ptr(w->gate_up, 16)) || (rc = check_ptr(w->down, 16))) return rc;
    if (d.wfmt != MOE_WFMT_BF16 && (!w->gate_up_scale || !w->down_scale)) return MOE_ERR_INVALID_ARG;
    if (d.wfmt == MOE_WFMT_MXFP4_PACKED && (!aligned(w->gate_up_scale, 8) || !aligned(w->down_scale, 8)))
        return MOE_ERR_MISALIGNED;
    return MOE_OK;
}

int check_ws(const moe_dims& d, const void* ws, size_t ws_bytes)
{
    if (ws_bytes < layout_for(d).total) return MOE_ERR_WORKSPACE;
    return check_ptr(ws, 16);
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return MOE_OK;
    g_last_error = hipGetErrorString(e);
    return MOE_ERR_HIP;
}

}  // namespace

void moe::set_last_error(const char* text) { g_last_error = text ? text : ""; }

namespace {

template <typename T>
T* region(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Skinny (weight streaming) while an expert can see at most this many tokens:
// per-expert token counts never exceed T, and up to 64 tokens the skinny
// kernels stay bound by weight traffic.
constexpr int kSkinnyMaxT = 64;

bool use_skinny(const moe_dims& d)
{
    if (d.path == MOE_PATH_SKINNY) return true;
    if (d.path != MOE_PATH_AUTO) return false;
    return d.T <= kSkinnyMaxT && (d.wfmt != MOE_WFMT_MXFP4_PACKED || packed_skinny_fits(d));
}

// Tiled regime on the MX matrix cores (MXFP4 weights; see MOE_PATH_TILED_MX):
// when asked for, and for TILED and AUTO in the tiled regime wherever it
// applies (on the 20b MXFP4 prefill it takes 0.82x the time of the
// bf16-decode kernel in the packed order, 0.97x row-major).
bool use_mx(const moe_dims& d)
{
    if (!mx_fits(d)) return false;
    return d.path == MOE_PATH_TILED_MX || d.path == MOE_PATH_TILED || (d.path == MOE_PATH_AUTO && !use_skinny(d));
}

moe::FfnArgs ffn_args(const moe_dims& d)
{
    moe::FfnArgs a;
    memset(&a, 0, sizeof a);
    a.T = d.T;
    a.H = d.H;
    a.E = d.E;
    a.k = d.k;
    a.I = d.I;
    a.wfmt = d.wfmt;
    return a;
}

// ---- stage bodies (arguments already validated) ----

int do_route(const moe_dims& d, const void* x, const void* wr, int32_t* idx, float* w, void* ws, hipStream_t s)
{
    const Layout L = layout_for(d);
    return hip_status(moe::launch_router_topk(d.T, d.H, d.E, d.k, static_cast<const uint16_t*>(x),
                                              static_cast<const uint16_t*>(wr), region<double>(ws, L.logits), idx, w,
                                              s));
}

// Route + permute.  For a handful of tokens selection and permutation run as
// one kernel after the logits kernel (one workgroup, one wave per token).
// With more tokens its waves select several tokens each in turn, and the
// parallel selection kernel followed by the permutation kernel is faster
// (per layer, same bits: 16 tokens -0.5 us, 64 tokens -10 us, 512 tokens
// -106 us; at 8 tokens the single kernel is 0.6 us faster).
constexpr int SELECT_PERMUTE_MAX_T = 8;

int do_route_permute(const moe_dims& d, const void* x, const void* wr, int32_t* idx, float* w, int32_t* off,
                     int32_t* sp, int32_t* pr, void* ws, hipStream_t s)
{
    if (d.T > SELECT_PERMUTE_MAX_T || !moe::permute_fits_one_block(d.T * d.k) ||
        moe::router_fuses_select(d.T, d.E)) {
        int rc = do_route(d, x, wr, idx, w, ws, s);
        if (rc) return rc;
        const Layout L = layout_for(d);
        return hip_status(moe::launch_permute(d.T * d.k, d.E, idx, off, sp, pr, region<void>(ws, L.perm_scratch), s));
    }
    const Layout L = layout_for(d);
    double* logits = region<double>(ws, L.logits);
    int rc = hip_status(moe::launch_router_logits_f64(d.T, d.H, d.E, static_cast<const uint16_t*>(x),
                                                      static_cast<const uint16_t*>(wr), logits, s));
    if (rc) return rc;
    return hip_status(moe::launch_select_permute_small(d.T, d.E, d.k, logits, idx, w, off, sp, pr, s));
}

int do_permute(const moe_dims& d, const int32_t* idx, int32_t* off, int32_t* sp, int32_t* pr, void* ws, hipStream_t s)
{
    const Layout L = layout_for(d);
    return hip_status(moe::launch_permute(d.T * d.k, d.E, idx, off, sp, pr, region<void>(ws, L.perm_scratch), s));
}

// The MX path splits the activations into the workspace first (x: T rows,
// h: P rows), then runs the MX grouped GEMM on them.  With h_split the MX
// gate/up kernel writes h already split (into the workspace regions that
// do_down reads with h_split) and no bf16 h at all; results are the same bits.
int do_gate_up(const moe_dims& d, const void* x, const int32_t* off, const int32_t* sp, const moe_expert_weights& w,
               void* h, void* ws, hipStream_t s, bool h_split = false)
{
    moe::FfnArgs a = ffn_args(d);
    a.x = static_cast<const uint16_t*>(x);
    a.offsets = off;
    a.sorted_pairs = sp;
    a.w = w.gate_up;
    a.w_scale = w.gate_up_scale;
    a.out = static_cast<uint16_t*>(h);
    if (use_mx(d)) {
        const Layout L = layout_for(d);
        a.a_codes = region<uint8_t>(ws, L.xs_codes);
        a.a_scales = region<uint8_t>(ws, L.xs_scales);
        if (h_split) {
            a.out_codes = region<uint8_t>(ws, L.hs_codes);
            a.out_scales = region<uint8_t>(ws, L.hs_scales);
        }
        int rc = hip_status(moe::launch_mx_split(a.x, d.T, d.H, region<uint8_t>(ws, L.xs_codes),
                                                 region<uint8_t>(ws, L.xs_scales), s));
        if (rc) return rc;
        return hip_status(moe::launch_gate_up_mx(a, s));
    }
    return hip_status(use_skinny(d) ? moe::launch_gate_up_skinny(a, s) : moe::launch_gate_up_tiled(a, s));
}

int do_down(const moe_dims& d, const void* h, const int32_t* off, const moe_expert_weights& w, void* ys, void* ws,
            hipStream_t s, bool h_split = false)
{
    moe::FfnArgs a = ffn_args(d);
    a.offsets = off;
    a.a_rows = static_cast<const uint16_t*>(h);
    a.w = w.down;
    a.w_scale = w.down_scale;
    a.out = static_cast<uint16_t*>(ys);
    if (use_mx(d)) {
        const Layout L = layout_for(d);
        a.a_codes = region<uint8_t>(ws, L.hs_codes);
        a.a_scales = region<uint8_t>(ws, L.hs_scales);
        if (!h_split) {
            int rc = hip_status(moe::launch_mx_split(a.a_rows, (int64_t)d.T * d.k, d.I,
                                                     region<uint8_t>(ws, L.hs_codes),
                                                     region<uint8_t>(ws, L.hs_scales), s));
            if (rc) return rc;
        }
        return hip_status(moe::launch_down_mx(a, s));
    }
    return hip_status(use_skinny(d) ? moe::launch_down_skinny(a, s) : moe::launch_down_tiled(a, s));
}

// Backward workspace: the forward's regions first (the stages reuse them),
// then the saved activations, the gradients in flight, the transposed
// weights and the per-expert transposed segments (Ppad rows each).
struct BwdLayout {
    size_t gu, dO, dw, da, dgu, dxp, padoff, dlT, wdT, wguT, dOT, hT, dguT, xT, rwp, total;
};

BwdLayout bwd_layout_for(const moe_dims& d)
{
    const size_t P = (size_t)d.T * (size_t)d.k, H = (size_t)d.H, I = (size_t)d.I, E = (size_t)d.E;
    const size_t Ppad = (size_t)moe::backward_pad_rows((int)P, d.E);
    BwdLayout L;
    size_t at = align_up(layout_for(d).total);
    auto take = [&](size_t bytes) {
        size_t here = at;
        at = align_up(at + bytes);
        return here;
    };
    L.gu = take(P * 2 * I * 2);
    L.dO = take(P * H * 2);
    L.dw = take(P * sizeof(float));
    L.da = take(P * I * 2);
    L.dgu = take(P * 2 * I * 2);
    L.dxp = take(P * H * 2);
    L.padoff = take((E + 1) * sizeof(int32_t));
    L.dlT = take(Ppad * 2);
    L.wdT = take(E * H * I * 2);
    L.wguT = take(E * 2 * I * H * 2);
    L.dOT = take(H * Ppad * 2);
    L.hT = take(I * Ppad * 2);
    L.dguT = take(2 * I * Ppad * 2);
    L.xT = take(H * Ppad * 2);
    L.rwp = take((size_t)moe::router_wgrad_splits((int)P, d.E) * H * sizeof(float));
    L.total = at;
    return L;
}

}  // namespace

extern "C" {

int moe_backward_workspace_size(const moe_dims* dims, size_t* bytes)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    if (dims->wfmt != MOE_WFMT_BF16) return MOE_ERR_UNSUPPORTED;
    *bytes = bwd_layout_for(*dims).total;
    return MOE_OK;
}

int moe_backward(const moe_dims* dims, const void* x, const void* w_router, const moe_expert_weights* weights,
                 const void* dy, void* dx, float* dw_router, float* dgate_up, float* ddown, void* workspace,
                 size_t workspace_bytes, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.wfmt != MOE_WFMT_BF16) return MOE_ERR_UNSUPPORTED;
    if (!dw_router || !dgate_up || !ddown) return MOE_ERR_INVALID_ARG;
    if (!aligned(dw_router, 4) || !aligned(dgate_up, 4) || !aligned(ddown, 4)) return MOE_ERR_MISALIGNED;
    if ((rc = check_weights(d, weights)) || (rc = check_ptr(w_router, 16))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const long long nr = (long long)d.E * d.H, ngu = (long long)d.E * 2 * d.I * d.H, nd = (long long)d.E * d.H * d.I;
    if (d.T == 0) {  // no tokens: every weight gradient is zero
        if ((rc = hip_status(moe::launch_zero_f32(dw_router, nr, s)))) return rc;
        if ((rc = hip_status(moe::launch_zero_f32(dgate_up, ngu, s)))) return rc;
        return hip_status(moe::launch_zero_f32(ddown, nd, s));
    }
    if ((rc = check_ptr(x, 16)) || (rc = check_ptr(dy, 16)) || (rc = check_ptr(dx, 16))) return rc;
    const BwdLayout B = bwd_layout_for(d);
    if (workspace_bytes < B.total) return MOE_ERR_WORKSPACE;
    if ((rc = check_ptr(workspace, 16))) return rc;
    const Layout L = layout_for(d);
    void* ws = workspace;
    const int P = d.T * d.k, H = d.H, I = d.I, E = d.E;
    int32_t* idx = region<int32_t>(ws, L.topk_idx);
    float* w = region<float>(ws, L.topk_w);
    int32_t* off = region<int32_t>(ws, L.offsets);
    int32_t* sp = region<int32_t>(ws, L.sorted);
    int32_t* pr = region<int32_t>(ws, L.rank);
    uint16_t* h = region<uint16_t>(ws, L.h);
    uint16_t* ys = region<uint16_t>(ws, L.y_sorted);
    uint16_t* gu = region<uint16_t>(ws, B.gu);
    uint16_t* dO = region<uint16_t>(ws, B.dO);
    float* dw = region<float>(ws, B.dw);
    uint16_t* da = region<uint16_t>(ws, B.da);
    uint16_t* dgu = region<uint16_t>(ws, B.dgu);
    uint16_t* dxp = region<uint16_t>(ws, B.dxp);
    int32_t* padoff = region<int32_t>(ws, B.padoff);
    uint16_t* dlT = region<uint16_t>(ws, B.dlT);
    uint16_t* wdT = region<uint16_t>(ws, B.wdT);
    uint16_t* wguT = region<uint16_t>(ws, B.wguT);
    uint16_t* dOT = region<uint16_t>(ws, B.dOT);
    uint16_t* hT = region<uint16_t>(ws, B.hT);
    uint16_t* dguT = region<uint16_t>(ws, B.dguT);
    uint16_t* xT = region<uint16_t>(ws, B.xT);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wgu = static_cast<const uint16_t*>(weights->gate_up);
    const uint16_t* wdn = static_cast<const uint16_t*>(weights->down);

    // forward, keeping g and u (tiled schedule: it is the one that stores them)
    if ((rc = do_route_permute(d, x, w_router, idx, w, off, sp, pr, ws, s))) return rc;
    moe::FfnArgs a = ffn_args(d);
    a.x = xb;
    a.offsets = off;
    a.sorted_pairs = sp;
    a.w = wgu;
    a.out = h;
    a.gu_out = gu;
    if ((rc = hip_status(moe::launch_gate_up_tiled(a, s)))) return rc;
    a = ffn_args(d);
    a.offsets = off;
    a.a_rows = h;
    a.w = wdn;
    a.out = ys;
    if ((rc = hip_status(moe::launch_down_tiled(a, s)))) return rc;
    // combine backward: dO = w dy per sorted row, dw = dy . o
    if ((rc = hip_status(moe::launch_combine_bwd(P, H, d.k, static_cast<const uint16_t*>(dy), ys, sp, w, dO, dw, s))))
        return rc;
    // data gradients on transposed weights, through the down-projection kernel
    if ((rc = hip_status(moe::launch_transpose_batched(wdn, wdT, E, H, I, s)))) return rc;      // [E][I][H]
    if ((rc = hip_status(moe::launch_transpose_batched(wgu, wguT, E, 2 * I, H, s)))) return rc;  // [E][H][2I]
    a = ffn_args(d);
    a.H = I;  // output width
    a.I = H;  // contracted width
    a.offsets = off;
    a.a_rows = dO;
    a.w = wdT;
    a.out = da;
    if ((rc = hip_status(moe::launch_down_tiled(a, s)))) return rc;
    if ((rc = hip_status(moe::launch_swiglu_bwd(P, I, da, gu, dgu, s)))) return rc;
    a = ffn_args(d);
    a.H = H;
    a.I = 2 * I;
    a.offsets = off;
    a.a_rows = dgu;
    a.w = wguT;
    a.out = dxp;
    if ((rc = hip_status(moe::launch_down_tiled(a, s)))) return rc;
    // router backward and dx
    if ((rc = hip_status(moe::launch_pad_offsets(off, E, padoff, dlT, s)))) return rc;
    if ((rc = hip_status(moe::launch_router_bwd(d.T, H, d.k, static_cast<const uint16_t*>(w_router), idx, w, dw, pr,
                                                off, padoff, dxp, dlT, static_cast<uint16_t*>(dx), s))))
        return rc;
    // weight gradients over each expert's transposed, zero-padded segment
    if ((rc = hip_status(moe::launch_transpose_segments(dO, H, false, off, padoff, sp, d.k, P, E, dOT, s)))) return rc;
    if ((rc = hip_status(moe::launch_transpose_segments(h, I, false, off, padoff, sp, d.k, P, E, hT, s)))) return rc;
    if ((rc = hip_status(moe::launch_transpose_segments(dgu, 2 * I, false, off, padoff, sp, d.k, P, E, dguT, s))))
        return rc;
    if ((rc = hip_status(moe::launch_transpose_segments(xb, H, true, off, padoff, sp, d.k, P, E, xT, s)))) return rc;
    if ((rc = hip_status(moe::launch_wgrad_tiled(dOT, hT, padoff, E, H, I, ddown, s)))) return rc;
    if ((rc = hip_status(moe::launch_wgrad_tiled(dguT, xT, padoff, E, 2 * I, H, dgate_up, s)))) return rc;
    return hip_status(moe::launch_router_wgrad(H, E, d.k, P, off, padoff, sp, dlT, xb, region<float>(ws, B.rwp),
                                               dw_router, s));
}

int moe_workspace_size(const moe_dims* dims, size_t* bytes)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = layout_for(*dims).total;
    return MOE_OK;
}

int moe_route(const moe_dims* dims, const void* x, const void* w_router, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(x, 16)) || (rc = check_ptr(w_router, 16)) || (rc = check_ptr(topk_idx, 4)) ||
        (rc = check_ptr(topk_w, 4)) || (rc = check_ws(d, workspace, workspace_bytes)))
        return rc;
    return do_route(d, x, w_router, topk_idx, topk_w, workspace, static_cast<hipStream_t>(stream));
}

int moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_offsets, int32_t* sorted_pairs,
                int32_t* pair_rank, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(topk_idx, 4)) || (rc = check_ptr(expert_offsets, 4)) || (rc = check_ptr(sorted_pairs, 4)) ||
        (rc = check_ptr(pair_rank, 4)) || (rc = check_ws(d, workspace, workspace_bytes)))
        return rc;
    return do_permute(d, topk_idx, expert_offsets, sorted_pairs, pair_rank, workspace,
                      static_cast<hipStream_t>(stream));
}

int moe_gate_up(const moe_dims* dims, const void* x, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                const moe_expert_weights* weights, void* h, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(x, 16)) || (rc = check_ptr(expert_offsets, 4)) || (rc = check_ptr(sorted_pairs, 4)) ||
        (rc = check_weights(d, weights)) || (rc = check_ptr(h, 16)))
        return rc;
    if (use_mx(d) && (rc = check_ws(d, workspace, workspace_bytes))) return rc;
    return do_gate_up(d, x, expert_offsets, sorted_pairs, *weights, h, workspace, static_cast<hipStream_t>(stream));
}

int moe_down(const moe_dims* dims, const void* h, const int32_t* expert_offsets, const moe_expert_weights* weights,
             void* y_sorted, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(h, 16)) || (rc = check_ptr(expert_offsets, 4)) || (rc = check_weights(d, weights)) ||
        (rc = check_ptr(y_sorted, 16)))
        return rc;
    if (use_mx(d) && (rc = check_ws(d, workspace, workspace_bytes))) return rc;
    return do_down(d, h, expert_offsets, *weights, y_sorted, workspace, static_cast<hipStream_t>(stream));
}

int moe_grouped_ffn(const moe_dims* dims, const void* x, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                    const moe_expert_weights* weights, void* y_sorted, void* workspace, size_t workspace_bytes,
                    void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(x, 16)) || (rc = check_ptr(expert_offsets, 4)) || (rc = check_ptr(sorted_pairs, 4)) ||
        (rc = check_weights(d, weights)) || (rc = check_ptr(y_sorted, 16)) ||
        (rc = check_ws(d, workspace, workspace_bytes)))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* h = region<void>(workspace, layout_for(d).h);
    if ((rc = do_gate_up(d, x, expert_offsets, sorted_pairs, *weights, h, workspace, s, true))) return rc;
    return do_down(d, h, expert_offsets, *weights, y_sorted, workspace, s, true);
}

int moe_combine(const moe_dims* dims, const void* y_sorted, const int32_t* pair_rank, const float* topk_w, void* y,
                void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(y_sorted, 16)) || (rc = check_ptr(pair_rank, 4)) || (rc = check_ptr(topk_w, 4)) ||
        (rc = check_ptr(y, 16)))
        return rc;
    return hip_status(moe::launch_combine(d.T, d.H, d.k, static_cast<const uint16_t*>(y_sorted), pair_rank, topk_w,
                                          static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream)));
}

int moe_forward(const moe_dims* dims, const void* x, const void* w_router, const moe_expert_weights* weights, void* y,
                int32_t* topk_idx_out, float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    const moe_dims& d = *dims;
    if (d.T == 0) return MOE_OK;
    if ((rc = check_ptr(x, 16)) || (rc = check_ptr(w_router, 16)) || (rc = check_weights(d, weights)) ||
        (rc = check_ptr(y, 16)) || (rc = check_ws(d, workspace, workspace_bytes)))
        return rc;
    if ((topk_idx_out && !aligned(topk_idx_out, 4)) || (topk_w_out && !aligned(topk_w_out, 4)))
        return MOE_ERR_MISALIGNED;
    const Layout L = layout_for(d);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* idx = topk_idx_out ? topk_idx_out : region<int32_t>(workspace, L.topk_idx);
    float* w = topk_w_out ? topk_w_out : region<float>(workspace, L.topk_w);
    int32_t* off = region<int32_t>(workspace, L.offsets);
    int32_t* sp = region<int32_t>(workspace, L.sorted);
    int32_t* pr = region<int32_t>(workspace, L.rank);
    void* h = region<void>(workspace, L.h);
    void* ys = region<void>(workspace, L.y_sorted);
    if ((rc = do_route_permute(d, x, w_router, idx, w, off, sp, pr, workspace, s))) return rc;
    if ((rc = do_gate_up(d, x, off, sp, *weights, h, workspace, s, true))) return rc;
    if ((rc = do_down(d, h, off, *weights, ys, workspace, s, true))) return rc;
    return hip_status(moe::launch_combine(d.T, d.H, d.k, static_cast<const uint16_t*>(ys), pr, w,
                                          static_cast<uint16_t*>(y), s));
}

namespace {

// Shared validation of the quantiser entry points.
int check_quant(int64_t rows, int32_t cols, const void* w, int64_t* n_elems)
{
    if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
    if (cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
    if (rows != 0 && cols != 0 && rows > moe::mxfp4_quant_max_elems() / cols) return MOE_ERR_UNSUPPORTED;
    *n_elems = rows * (int64_t)cols;
    if (*n_elems == 0) return MOE_OK;
    return check_ptr(w, 16);
}

}  // namespace

int moe_mxfp4_quantize(int64_t rows, int32_t cols, const void* w, uint8_t* packed, uint8_t* scales, void* stream)
{
    int64_t n = 0;
    int rc = check_quant(rows, cols, w, &n);
    if (rc || n == 0) return rc;
    if ((rc = check_ptr(packed, 16))) return rc;
    if (!scales) return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_mxfp4_quantize(static_cast<const uint16_t*>(w), n, packed, scales,
                                                 static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_pack(const moe_dims* dims, int32_t which, const uint8_t* w, const uint8_t* scales, uint8_t* w_packed,
                   uint8_t* scales_packed, void* stream)
{
    int rc = check_dims(dims);
    if (rc) return rc;
    if (which != MOE_PACK_GATE_UP && which != MOE_PACK_DOWN) return MOE_ERR_INVALID_ARG;
    if (!scales) return MOE_ERR_INVALID_ARG;
    if ((rc = check_ptr(w, 16)) || (rc = check_ptr(w_packed, 16)) || (rc = check_ptr(scales_packed, 8))) return rc;
    const bool gu = which == MOE_PACK_GATE_UP;
    const int64_t R = gu ? 2 * (int64_t)dims->I : dims->H, K = gu ? dims->H : dims->I;
    const int64_t bytes = (int64_t)dims->E * R * (K / 2), sbytes = (int64_t)dims->E * R * (K / 32);
    auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
        const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
        return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
    };
    if (overlap(w_packed, bytes, w, bytes) || overlap(w_packed, bytes, scales, sbytes) ||
        overlap(scales_packed, sbytes, w, bytes) || overlap(scales_packed, sbytes, scales, sbytes) ||
        overlap(w_packed, bytes, scales_packed, sbytes))
        return MOE_ERR_INVALID_ARG;
    return hip_status(moe::launch_mxfp4_pack(gu, dims->E, dims->I, dims->H, w, scales, w_packed, scales_packed,
                                             static_cast<hipStream_t>(stream)));
}

int moe_mx_split(int64_t rows, int32_t cols, const void* x, uint8_t* codes, uint8_t* scales, void* stream)
{
    if (rows < 0) return MOE_ERR_INVALID_ARG;
    if (cols <= 0 || cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    int rc;
    if ((rc = check_ptr(x, 16)) || (rc = check_ptr(codes, 16)) || (rc = check_ptr(scales, 2))) return rc;
    return hip_status(moe::launch_mx_split(static_cast<const uint16_t*>(x), rows, cols, codes, scales,
                                           static_cast<hipStream_t>(stream)));
}

int moe_mxfp4_fakequant(int64_t rows, int32_t cols, const void* w, void* out, void* stream)
{
    int64_t n = 0;
    int rc = check_quant(rows, cols, w, &n);
    if (rc || n == 0) return rc;
    if ((rc = check_ptr(out, 16))) return rc;
    return hip_status(moe::launch_mxfp4_fakequant(static_cast<const uint16_t*>(w), n, static_cast<uint16_t*>(out),
                                                  static_cast<hipStream_t>(stream)));
}

const char* moe_strerror(int code)
{
    switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or format";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown error";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
