// aux_kernels.hip -- small kernels around the estimator scans: workspace
// fill, the debug data checks, and the bare wave-scan primitive exported for
// layout tests.
#include <atomic>
#include <mutex>

#include "rlscan_internal.hpp"
#include "scan_core.hpp"

namespace rlscan {

__global__ void debug_wave_scan_kernel(const float* a, const float* b, float* oa, float* ob) {
    const size_t i = (size_t)blockIdx.x * kWave + threadIdx.x;
    const Affine r = wave_inclusive_scan(Affine{a[i], b[i]});
    oa[i] = r.a;
    ob[i] = r.b;
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Data-contract checks (debug path, not tuned): one grid-stride pass over the
// flat [E,T] range, per-thread counts reduced in LDS, one global atomic per
// workgroup and counter, and only when that count is nonzero.
__global__ void check_kernel(const float* term, const float* trunc, const float* boot,
                             const int64_t* actions, int64_t N, int64_t T, int64_t A,
                             unsigned long long* counts) {
    unsigned long long c[4] = {0, 0, 0, 0};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < N;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float te = term ? term[i] : 0.f;
        const float tr = trunc ? trunc[i] : 0.f;
        if (term && !(te == 0.f || te == 1.f)) c[0]++;
        if (trunc && !(tr == 0.f || tr == 1.f)) c[0]++;
        if (term && trunc && te != 0.f && tr != 0.f) c[1]++;
        if (trunc && boot && tr == 0.f && (i % T) != T - 1 && boot[i] != 0.f) c[2]++;
        if (actions) {
            const int64_t a = actions[i];
            if (a < 0 || a >= A) c[3]++;
        }
    }
    __shared__ unsigned long long s_counts[4];
    if (threadIdx.x < 4) s_counts[threadIdx.x] = 0;
    __syncthreads();
    for (int k = 0; k < 4; ++k)
        if (c[k]) atomicAdd(&s_counts[k], c[k]);
    __syncthreads();
    if (threadIdx.x < 4 && s_counts[threadIdx.x]) atomicAdd(&counts[threadIdx.x], s_counts[threadIdx.x]);
}

// Streaming reference for the roofline context: NIN fp32 arrays read and
// NOUT written per element, with the scan kernels' access pattern and launch
// shape but no scan (512-thread workgroups, tiles of two 1 KiB-per-wave
// segments, 16-byte non-temporal loads all issued before any store, the same
// pause between segments, plain 16-byte stores).  Its time for a workload's
// arrays is what the memory system gives that pattern on this device.
constexpr int kStreamMax = 6;
constexpr int kStreamTile = 4096;
struct StreamPtrs {
    const float* in[kStreamMax];
    float* out[kStreamMax];
};

template <int NIN, int NOUT>
__global__ __launch_bounds__(512) void stream_kernel(StreamPtrs p) {
    const size_t t0 = (size_t)blockIdx.x * kStreamTile;
    const size_t base = t0 + threadIdx.x * 4;  // segment 0
    f32x4 v[2][NIN];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int a = 0; a < NIN; ++a) v[s][a] = load16(p.in[a] + base + s * (kStreamTile / 2));
        if (s == 0) __builtin_amdgcn_s_sleep(4);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        f32x4 acc = v[s][0];
#pragma unroll
        for (int a = 1; a < NIN; ++a) acc += v[s][a];
#pragma unroll
        for (int o = 0; o < NOUT; ++o)
            store16<true>(p.out[o] + t0, (uint32_t)(threadIdx.x * 4 + s * (kStreamTile / 2)) * 4u,
                          kStreamTile * 4u, acc);
    }
}

template <int NIN, int NOUT>
static void launch_stream_n(const StreamPtrs& p, int64_t n, hipStream_t s) {
    hipLaunchKernelGGL((stream_kernel<NIN, NOUT>), dim3((unsigned)(n / kStreamTile)), dim3(512), 0,
                       s, p);
}

rlscan_status launch_debug_stream(const float* const* in, int nin, float* const* out, int nout,
                                  int64_t n, hipStream_t s) {
    StreamPtrs p{};
    for (int a = 0; a < nin; ++a) p.in[a] = in[a];
    for (int o = 0; o < nout; ++o) p.out[o] = out[o];
    switch (nin * 10 + nout) {
        case 11: launch_stream_n<1, 1>(p, n, s); break;
        case 21: launch_stream_n<2, 1>(p, n, s); break;
        case 31: launch_stream_n<3, 1>(p, n, s); break;
        case 41: launch_stream_n<4, 1>(p, n, s); break;
        case 42: launch_stream_n<4, 2>(p, n, s); break;
        case 52: launch_stream_n<5, 2>(p, n, s); break;
        case 62: launch_stream_n<6, 2>(p, n, s); break;
        default: return set_error(RLSCAN_ERR_BAD_PARAM, "unsupported number of input/output arrays");
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

rlscan_status launch_debug_wave_scan(const float* a, const float* b, float* oa, float* ob,
                                     int num_waves, hipStream_t s) {
    hipLaunchKernelGGL(debug_wave_scan_kernel, dim3((unsigned)num_waves), dim3(kWave), 0, s, a, b,
                       oa, ob);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

rlscan_status launch_check(const float* term, const float* trunc, const float* boot,
                           const int64_t* actions, int64_t N, int64_t T, int64_t A,
                           unsigned long long* counts, hipStream_t s) {
    int64_t blocks = (N + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, term, trunc, boot,
                       actions, N, T, A, counts);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

int resident_workgroups(const void* kernel, int threads) {
    // Small fixed cache: (kernel, device) -> workgroups resident at once.
    struct Entry {
        const void* kernel;
        int device;
        int count;
    };
    static Entry cache[256];
    static std::atomic<int> used{0};
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int n = used.load(std::memory_order_acquire);
    for (int i = 0; i < n; ++i)
        if (cache[i].kernel == kernel && cache[i].device == dev) return cache[i].count;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;  // unknown: treated as "not resident at once"
    }
    const int count = per_cu * cus;
    std::lock_guard<std::mutex> lock(mu);
    const int m = used.load(std::memory_order_relaxed);
    if (m < 256) {
        cache[m] = Entry{kernel, dev, count};
        used.store(m + 1, std::memory_order_release);
    }
    return count;
}

rlscan_status launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t words = bytes / 4;
    if (words == 0) return RLSCAN_OK;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(p), words);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
    return RLSCAN_OK;
}

}  // namespace rlscan
