// op_gae_norm.hip -- GAE with batch advantage normalisation (paper Sec. 9.3
// plans fused advantage normalisation; the formula is the usual whitening of
// PPO advantages):
//   adv_t = (A_t - mean) / (std + eps),  mean and unbiased std over all E*T steps.
// Three launches on the stream:
//   1. the GAE scan, whose tiles also reduce their advantages to a
//      (count, mean, M2) triple in the workspace (scan_tile's statistics);
//   2. one workgroup merges the triples in a fixed order in double precision
//      (Chan et al.'s pairwise update), so the statistics are reproducible;
//   3. an elementwise pass normalises the advantages in place.
// Pass 3 re-reads and rewrites the advantages: 8 more bytes per step than the
// plain GAE call, against the separate mean, std and normalisation passes
// (at least 16 bytes per step) it replaces.
#include <algorithm>

#include "op_gae.hpp"

namespace rlscan {

namespace {

struct StatD {
    double n, m, m2;
};

__device__ __forceinline__ StatD merge_d(StatD a, StatD b) {
    const double n = a.n + b.n;
    if (n == 0.0) return StatD{0.0, 0.0, 0.0};
    const double d = b.m - a.m;
    const double w = b.n / n;
    return StatD{n, a.m + d * w, a.m2 + b.m2 + d * d * a.n * w};
}

constexpr int kFinalThreads = 1024;
constexpr int kFinalBatch = 4;  // triples a thread loads before merging them

// result[0] = mean, result[1] = std (unbiased; 0 for one step),
// result[2] = 1 / (std + eps).
__global__ __launch_bounds__(kFinalThreads) void stats_finalize_kernel(const double* tiles,
                                                                       int64_t num_tiles,
                                                                       double eps, double* result,
                                                                       double* user) {
    __shared__ StatD sh[kFinalThreads];
    const int i = threadIdx.x;
    // thread i merges tiles i, i + 1024, i + 2048, ... in that order; the
    // loads of a batch are all issued before the first merge
    StatD acc{0.0, 0.0, 0.0};
    for (int64_t t0 = i; t0 < num_tiles; t0 += (int64_t)kFinalBatch * kFinalThreads) {
        StatD b[kFinalBatch];
#pragma unroll
        for (int u = 0; u < kFinalBatch; ++u) {
            const int64_t t = t0 + (int64_t)u * kFinalThreads;
            b[u] = t < num_tiles ? StatD{tiles[4 * t], tiles[4 * t + 1], tiles[4 * t + 2]}
                                 : StatD{0.0, 0.0, 0.0};
        }
#pragma unroll
        for (int u = 0; u < kFinalBatch; ++u) acc = merge_d(acc, b[u]);
    }
    sh[i] = acc;
    __syncthreads();
    for (int stride = kFinalThreads / 2; stride >= 1; stride >>= 1) {
        if (i < stride) sh[i] = merge_d(sh[i], sh[i + stride]);
        __syncthreads();
    }
    if (i == 0) {
        const StatD s = sh[0];
        const double sd = s.n > 1.0 ? sqrt(s.m2 / (s.n - 1.0)) : 0.0;
        result[0] = s.m;
        result[1] = sd;
        result[2] = 1.0 / (sd + eps);
        if (user) {
            user[0] = s.m;
            user[1] = sd;
        }
    }
}

// Four consecutive advantages per thread and step of a grid-stride loop
// (16-byte accesses when aligned).
__global__ __launch_bounds__(256) void normalize_kernel(float* adv, int64_t n, const double* result,
                                                        int vec) {
    const float mean = (float)result[0];
    const float inv = (float)result[2];
    const int64_t stride = (int64_t)gridDim.x * 256 * 4;
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += stride) {
        if (vec && i + 4 <= n) {
            f32x4 v = *reinterpret_cast<const f32x4*>(adv + i);
            v.x = (v.x - mean) * inv;
            v.y = (v.y - mean) * inv;
            v.z = (v.z - mean) * inv;
            v.w = (v.w - mean) * inv;
            *reinterpret_cast<f32x4*>(adv + i) = v;
        } else {
            for (int64_t j = i; j < i + 4 && j < n; ++j) adv[j] = (adv[j] - mean) * inv;
        }
    }
}

rlscan_status last_launch_status() {
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? RLSCAN_OK : set_error(RLSCAN_ERR_LAUNCH, hipGetErrorString(err));
}

}  // namespace

rlscan_status launch_gae_norm(const GaeArgs& args, const Plan& plan, void* ws, size_t stats_off,
                              int64_t N, float eps, double* stats_out, hipStream_t s) {
    GaeArgs a = args;
    double* tiles = reinterpret_cast<double*>(static_cast<uint8_t*>(ws) + stats_off);
    double* result = tiles + 4 * plan.geo.num_tiles;
    a.tile_stats = tiles;
    rlscan_status st;
    if (!a.truncateds)
        st = launch_gae_op<kStatsOut>(a, plan, ws, s);
    else if (!a.bootstrap_values)
        st = launch_gae_op<kStatsOut | kTrunc>(a, plan, ws, s);
    else
        st = launch_gae_op<kStatsOut | kTrunc | kBoot2D>(a, plan, ws, s);
    if (st != RLSCAN_OK) return st;
    hipLaunchKernelGGL(stats_finalize_kernel, dim3(1), dim3(kFinalThreads), 0, s, tiles,
                       plan.geo.num_tiles, (double)eps, result, stats_out);
    if ((st = last_launch_status()) != RLSCAN_OK) return st;
    const int64_t blocks = std::min<int64_t>((N + 1023) / 1024, (int64_t)1 << 20);
    const int vec = (reinterpret_cast<uintptr_t>(a.advantages) & 15u) == 0;
    hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.advantages, N,
                       result, vec);
    return last_launch_status();
}

}  // namespace rlscan
