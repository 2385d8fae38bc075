// moe_forward_noalloc: the whole layer with its workspace in a library-owned
// device array instead of a caller-provided buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The kernels and their order are
// moe_forward's; only where the intermediates live differs.
//
// The array is a file-scope __device__ variable, so each GPU the library runs
// on holds its own copy (MOE_NOALLOC_SCRATCH_BYTES) from module load until
// the process ends.  Host code may not pass the array's name to a kernel (on
// the host it is only a stand-in for the symbol): its device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and that address is what the forward receives.
#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null until looked up)

// Device address of this device's `scratch`, looked up on first use.
int scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) return MOE_ERR_UNSUPPORTED;
    if (e == hipSuccess) {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (!g_scratch_ptr[dev]) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e == hipSuccess) g_scratch_ptr[dev] = p;
        }
        *out = g_scratch_ptr[dev];
    }
    if (e != hipSuccess) {
        moe::set_last_error(hipGetErrorString(e));
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const moe_dims* dims, const void* x, const void* w_router, const moe_expert_weights* weights,
                        void* y, int32_t* topk_idx_out, float* topk_w_out, void* stream)
{
    size_t need = 0;
    int rc = moe_workspace_size(dims, &need);
    if (rc) return rc;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    if (dims->T == 0) return MOE_OK;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return moe_forward(dims, x, w_router, weights, y, topk_idx_out, topk_w_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                       stream);
}

}  // extern "C"
