// noalloc.hip -- rlscan_gae_noalloc: rlscan_gae with its look-back workspace
// in a static device array of the library instead of a caller-provided
// buffer, for callers that cannot allocate device memory.
//
// The array below is a file-scope device symbol: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never uses the symbol's name as an address (in host code it names a
// host-side stand-in); it takes the device address that hipGetSymbolAddress
// returns, once per device, and passes that pointer to the kernels and to the
// fill kernel, exactly as it passes a caller's workspace in rlscan_gae.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rlscan_internal.hpp"

namespace rlscan {
namespace {

// 2 MiB: the 4352-byte header plus 32 bytes per tile, i.e. room for 65,400
// look-back tiles (about 268 million steps in 4096-step tiles).
constexpr size_t kScratchBytes = (size_t)2 << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of this device's `scratch` (the current device), set up on
// the first call on the device: the address is looked up with the device
// current, checked, kept, and the array is zero-filled on `stream` by the
// library's fill kernel (ordered before the call's own kernel).
rlscan_status device_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(RLSCAN_ERR_LAUNCH, "device index beyond the static scratch table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess || ptr == nullptr)
            return set_error(RLSCAN_ERR_LAUNCH, err != hipSuccess ? hipGetErrorString(err)
                                                                  : "scratch has no device address");
        const rlscan_status st = launch_fill_zero(ptr, kScratchBytes, stream);
        if (st != RLSCAN_OK) return st;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return RLSCAN_OK;
}

}  // namespace
}  // namespace rlscan

using namespace rlscan;

extern "C" rlscan_status rlscan_gae_noalloc(const float* rewards, const float* values,
                                            const float* terminateds, const float* truncateds,
                                            const float* bootstrap_values, const float* last_value,
                                            float* advantages, float* returns, int64_t num_envs,
                                            int64_t seq_len, float gamma, float lambda,
                                            rlscan_stream_t stream) {
    GaeArgs a;
    Plan plan;
    bool empty = false;
    const rlscan_status st =
        gae_prepare(rewards, values, terminateds, truncateds, bootstrap_values, last_value, nullptr,
                    advantages, returns, num_envs, seq_len, gamma, lambda, a, plan, empty);
    if (st != RLSCAN_OK || empty) return st;
    const size_t need = plan_workspace_bytes(plan);
    if (need > kScratchBytes)
        return set_error(RLSCAN_ERR_BAD_SHAPE,
                         "rlscan_gae_noalloc: this shape needs more look-back scratch than the "
                         "library's static 2 MiB (use rlscan_gae with a workspace)");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (need > 0) {
        const rlscan_status sst = device_scratch(s, &ws);
        if (sst != RLSCAN_OK) return sst;
    }
    return launch_gae(a, plan, ws, s);
}
