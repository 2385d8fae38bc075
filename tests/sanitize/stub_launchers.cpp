// Host-only stand-ins for the kernel launchers of moe_kernels.h, so that the
// C-ABI layer (moe_api.hip, compiled as plain C++) can be built and driven
// under AddressSanitizer and UndefinedBehaviorSanitizer on a machine without
// a GPU.  Test infrastructure: every launcher only counts the call and
// returns success; the size helpers follow the library's formulas closely
// enough for validation (they are the same functions the workspace-size
// entry points call, so sizes stay consistent).
#include "moe_kernels.h"

extern "C" {
long long stub_launches = 0;
}

namespace moe {

static hipError_t count() { ++stub_launches; return hipSuccess; }

hipError_t launch_router_logits_f64(int, int, int, const uint16_t*, const uint16_t*, double*, hipStream_t) { return count(); }
hipError_t launch_router_select(int, int, int, const double*, int32_t*, float*, hipStream_t) { return count(); }
bool router_fuses_select(int T, int E) { return T >= 1024 && E <= 64; }
hipError_t launch_router_topk(int, int, int, int, const uint16_t*, const uint16_t*, double*, int32_t*, float*,
                              hipStream_t) { return count(); }
size_t permute_scratch_bytes(int64_t P, int E) { return (size_t)(P + (P + 1023) / 1024 * E) * 4; }
hipError_t launch_permute(int, int, const int32_t*, int32_t*, int32_t*, int32_t*, void*, hipStream_t) { return count(); }
bool permute_fits_one_block(int P) { return P <= 4096; }
hipError_t launch_select_permute_small(int, int, int, const double*, int32_t*, float*, int32_t*, int32_t*, int32_t*,
                                       hipStream_t) { return count(); }
hipError_t launch_gate_up_skinny(const FfnArgs&, hipStream_t) { return count(); }
bool skinny4_supported(const FfnArgs& a)
{
    const long long lim = 1ll << 31, P = (long long)a.T * a.k;
    return (long long)a.I * a.H < lim && (long long)a.T * a.H * 2 < lim && P * a.I * 2 < lim && P * 4 < lim;
}
hipError_t launch_down_skinny(const FfnArgs&, hipStream_t) { return count(); }
hipError_t launch_gate_up_tiled(const FfnArgs&, hipStream_t) { return count(); }
hipError_t launch_down_tiled(const FfnArgs&, hipStream_t) { return count(); }
hipError_t launch_mx_split(const uint16_t*, int64_t, int, uint8_t*, uint8_t*, hipStream_t) { return count(); }
bool mx_supported(int H, int I) { return H % 64 == 0 && I % 64 == 0; }
hipError_t launch_gate_up_mx(const FfnArgs&, hipStream_t) { return count(); }
hipError_t launch_down_mx(const FfnArgs&, hipStream_t) { return count(); }
hipError_t launch_combine(int, int, int, const uint16_t*, const int32_t*, const float*, uint16_t*, hipStream_t) { return count(); }
int backward_pad_rows(int P, int E) { return P + 64 * E; }
hipError_t launch_zero_f32(float*, long long, hipStream_t) { return count(); }
hipError_t launch_transpose_batched(const uint16_t*, uint16_t*, int, int, int, hipStream_t) { return count(); }
hipError_t launch_pad_offsets(const int32_t*, int, int32_t*, uint16_t*, hipStream_t) { return count(); }
hipError_t launch_transpose_segments(const uint16_t*, int, bool, const int32_t*, const int32_t*, const int32_t*, int,
                                     int, int, uint16_t*, hipStream_t) { return count(); }
hipError_t launch_wgrad_tiled(const uint16_t*, const uint16_t*, const int32_t*, int, int, int, float*, hipStream_t) { return count(); }
long long router_wgrad_splits(int P, int E) { return ((long long)P + 63LL * E) / 64; }
hipError_t launch_router_wgrad(int, int, int, int, const int32_t*, const int32_t*, const int32_t*, const uint16_t*,
                               const uint16_t*, float*, float*, hipStream_t) { return count(); }
hipError_t launch_combine_bwd(int, int, int, const uint16_t*, const uint16_t*, const int32_t*, const float*, uint16_t*,
                              float*, hipStream_t) { return count(); }
hipError_t launch_swiglu_bwd(int, int, const uint16_t*, const uint16_t*, uint16_t*, hipStream_t) { return count(); }
hipError_t launch_router_bwd(int, int, int, const uint16_t*, const int32_t*, const float*, const float*, const int32_t*,
                             const int32_t*, const int32_t*, const uint16_t*, uint16_t*, uint16_t*, hipStream_t) { return count(); }
int64_t mxfp4_quant_max_elems() { return 1ll << 41; }
hipError_t launch_mxfp4_quantize(const uint16_t*, int64_t, uint8_t*, uint8_t*, hipStream_t) { return count(); }
hipError_t launch_mxfp4_fakequant(const uint16_t*, int64_t, uint16_t*, hipStream_t) { return count(); }
hipError_t launch_mxfp4_pack(bool, int, int, int, const uint8_t*, const uint8_t*, uint8_t*, uint8_t*, hipStream_t) { return count(); }

}  // namespace moe

// The HIP runtime's error text (the only runtime call the C-ABI layer makes).
const char* hipGetErrorString(hipError_t) { return "stub"; }
