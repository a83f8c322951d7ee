// op_gae_norm.hip -- GAE with batch advantage normalisation (paper Sec. 9.3
// plans fused advantage normalisation; the formula is the usual whitening of
// PPO advantages):
//   adv_t = (A_t - mean) / (std + eps),  mean and unbiased std over all E*T steps.
// Two launches on the stream:
//   1. the GAE scan, whose tiles also reduce their advantages to a
//      (count, mean, M2) triple in the workspace (scan_tile's statistics);
//   2. an elementwise pass that normalises the advantages in place.  Each of
//      its workgroups first issues the loads of its first chunk of
//      advantages, then combines all tile triples itself, in double precision
//      and one fixed order (batch_stats), so every workgroup holds the same
//      statistics bit for bit and they are reproducible.
// Above kFusedMaxTiles tiles the redundant work would cost more than a
// launch, and one workgroup combines the triples in a launch of its own
// between the two.  Pass 2 re-reads and rewrites the advantages: 8 more bytes per step
// than the plain GAE call, against the separate mean, std and normalisation
// passes (at least 16 bytes per step) it replaces.
#include <algorithm>

#include "op_gae.hpp"

namespace rlscan {

namespace {

struct StatD {
    double n, m, m2;
};

constexpr int kStatThreads = 1024;  // threads of every kernel that merges the triples
constexpr int kStatWaves = kStatThreads / 64;
constexpr int kStatBatch = 4;       // triples a thread loads before adding them
constexpr int64_t kFusedMaxTiles = 8192;

// Tile t's triple, or the empty triple past the last tile.  The load itself
// is unconditional (of tile 0 when t is out of range; num_tiles >= 1) and the
// out-of-range triple is zeroed by a multiply, not a branch, so a batch of
// loads is issued without waiting on any of them.  The triples are finite, so
// the multiply by 0 gives zeros.
__device__ __forceinline__ StatD load_triple(const double* tiles, int64_t t, int64_t num_tiles) {
    const bool in = t < num_tiles;
    const int64_t u = in ? t : 0;
    const double keep = (double)(int)in;
    return StatD{tiles[4 * u] * keep, tiles[4 * u + 1] * keep, tiles[4 * u + 2] * keep};
}

// Thread i's first batch: tiles i, i + 1024, i + 2048, i + 3072.
__device__ __forceinline__ void load_first_batch(const double* tiles, int64_t num_tiles,
                                                 StatD (&b)[kStatBatch]) {
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u)
        b[u] = load_triple(tiles, threadIdx.x + (int64_t)u * kStatThreads, num_tiles);
}

// x from the lane that the DPP control CTRL names, both 32-bit halves moved
// by the same pattern.
template <int CTRL>
__device__ __forceinline__ double dpp_move(double x) {
    const long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ double lane_value(double x, int lane) {
    const long long u = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readlane((int)u, lane);
    const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Sum over the 64 lanes of a wave, the same value in every lane: within each
// row of 16 lanes, swaps of neighbours and of pairs (quad permutations) and
// rotations by 4 and 8 lanes leave the row's sum in its lane 0; the four row
// sums are then added in row order.  A fixed order: the same bits on every
// call.
__device__ __forceinline__ double wave_sum(double x) {
    x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_move<0x124>(x);  // row_ror:4
    x += dpp_move<0x128>(x);  // row_ror:8
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

// Workgroup totals of x[0..K) over its kStatThreads threads; every thread
// gets them.  The wave sums (wave_sum) are added in wave order: the same
// bits on every call.
template <int K>
__device__ __forceinline__ void block_sum(double (&x)[K], double (&sh)[K][kStatWaves]) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] = wave_sum(x[k]);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int k = 0; k < K; ++k) sh[k][w] = x[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        x[k] = 0.0;
#pragma unroll
        for (int v = 0; v < kStatWaves; ++v) x[k] += sh[k][v];
    }
    __syncthreads();
}

struct BatchStats {
    double mean, sd;  // sd: unbiased, 0 for a one-step batch
};

// Batch mean and std from the tiles' (count n, mean m, M2) triples, by the
// decomposition of the sum of squares about the batch mean:
//   N = sum n_t,  mean = sum n_t m_t / N,  M2 = sum (M2_t + n_t (m_t - mean)^2).
// Every term of the last sum is non-negative, so nothing cancels, and no
// division is needed per tile.  Thread i takes tiles i, i + 1024, ... in
// turn, its first batch already loaded into `first`; later batches are read
// again for the second sum.
__device__ BatchStats batch_stats(const double* tiles, int64_t num_tiles,
                                  const StatD (&first)[kStatBatch],
                                  double (&sh)[2][kStatWaves]) {
    const int64_t step = (int64_t)kStatBatch * kStatThreads;
    double ns[2] = {0.0, 0.0};  // count, sum of n m
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u) {
        ns[0] += first[u].n;
        ns[1] = fma(first[u].n, first[u].m, ns[1]);
    }
    for (int64_t t0 = threadIdx.x + step; t0 < num_tiles; t0 += step) {
        StatD b[kStatBatch];
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) b[u] = load_triple(tiles, t0 + u * kStatThreads, num_tiles);
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) {
            ns[0] += b[u].n;
            ns[1] = fma(b[u].n, b[u].m, ns[1]);
        }
    }
    block_sum<2>(ns, sh);
    const double mean = ns[1] / ns[0];
    double q[1] = {0.0};
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u) {
        const double d = first[u].m - mean;
        q[0] += fma(first[u].n * d, d, first[u].m2);
    }
    for (int64_t t0 = threadIdx.x + step; t0 < num_tiles; t0 += step) {
        StatD b[kStatBatch];
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) b[u] = load_triple(tiles, t0 + u * kStatThreads, num_tiles);
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) {
            const double d = b[u].m - mean;
            q[0] += fma(b[u].n * d, d, b[u].m2);
        }
    }
    double (&sh1)[1][kStatWaves] = *reinterpret_cast<double (*)[1][kStatWaves]>(&sh[0][0]);
    block_sum<1>(q, sh1);
    return BatchStats{mean, ns[0] > 1.0 ? sqrt(q[0] / (ns[0] - 1.0)) : 0.0};
}

// One workgroup of kStatThreads threads.  result[0] = mean, result[1] = std,
// result[2] = 1 / (std + eps).
__global__ __launch_bounds__(kStatThreads) void stats_finalize_kernel(const double* tiles,
                                                                      int64_t num_tiles,
                                                                      double eps, double* result,
                                                                      double* user) {
    __shared__ double sh[2][kStatWaves];
    StatD first[kStatBatch];
    load_first_batch(tiles, num_tiles, first);
    const BatchStats st = batch_stats(tiles, num_tiles, first, sh);
    if (threadIdx.x == 0) {
        result[0] = st.mean;
        result[1] = st.sd;
        result[2] = 1.0 / (st.sd + eps);
        if (user) {
            user[0] = st.mean;
            user[1] = st.sd;
        }
    }
}

// ---- one launch: statistics merged by every workgroup, then normalisation ----
constexpr int kNormThreads = kStatThreads;
constexpr int kNormVecs = 4;  // groups of four advantages per thread and chunk
constexpr int64_t kNormChunk = (int64_t)kNormThreads * kNormVecs * 4;
constexpr int kNormMaxBlocks = 256;

// A thread's sixteen advantages of one chunk: group k is the four consecutive
// steps at base + 4 (k * kNormThreads + thread) when VEC (16-byte accesses),
// else element k * kNormThreads + thread for k < 16.
template <bool VEC>
struct NormChunk {
    float v[kNormVecs * 4];

    __device__ __forceinline__ int64_t index(int64_t base, int k, int c) const {
        return VEC ? base + ((int64_t)k * kNormThreads + threadIdx.x) * 4 + c
                   : base + (int64_t)(4 * k + c) * kNormThreads + threadIdx.x;
    }

    __device__ __forceinline__ void load(const float* adv, int64_t base, int64_t n) {
#pragma unroll
        for (int k = 0; k < kNormVecs; ++k) {
            const int64_t i = index(base, k, 0);
            if (VEC && i + 4 <= n) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(adv + i);
                v[4 * k] = x.x;
                v[4 * k + 1] = x.y;
                v[4 * k + 2] = x.z;
                v[4 * k + 3] = x.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t j = index(base, k, c);
                    v[4 * k + c] = j < n ? adv[j] : 0.f;
                }
            }
        }
    }

    __device__ __forceinline__ void store(float* adv, int64_t base, int64_t n, float mean,
                                          float inv) const {
#pragma unroll
        for (int k = 0; k < kNormVecs; ++k) {
            const int64_t i = index(base, k, 0);
            if (VEC && i + 4 <= n) {
                f32x4 x;
                x.x = (v[4 * k] - mean) * inv;
                x.y = (v[4 * k + 1] - mean) * inv;
                x.z = (v[4 * k + 2] - mean) * inv;
                x.w = (v[4 * k + 3] - mean) * inv;
                *reinterpret_cast<f32x4*>(adv + i) = x;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t j = index(base, k, c);
                    if (j < n) adv[j] = (v[4 * k + c] - mean) * inv;
                }
            }
        }
    }
};

// Every workgroup computes the batch statistics from all num_tiles triples
// (batch_stats: the same bits in every workgroup).  The loads of its first
// chunk of advantages are issued right after the first batch of triples, so
// their latency overlaps the two sums.
template <bool VEC>
__global__ __launch_bounds__(kNormThreads) void normalize_fused_kernel(
    float* adv, int64_t n, const double* tiles, int64_t num_tiles, double eps, double* user) {
    __shared__ double sh[2][kStatWaves];
    StatD first[kStatBatch];
    load_first_batch(tiles, num_tiles, first);
    int64_t base = (int64_t)blockIdx.x * kNormChunk;
    NormChunk<VEC> c;
    c.load(adv, base, n);
    const BatchStats st = batch_stats(tiles, num_tiles, first, sh);
    if (user && blockIdx.x == 0 && threadIdx.x == 0) {
        user[0] = st.mean;
        user[1] = st.sd;
    }
    const float mean = (float)st.mean;
    const float inv = (float)(1.0 / (st.sd + eps));
    const int64_t stride = (int64_t)gridDim.x * kNormChunk;
    for (;;) {
        c.store(adv, base, n, mean, inv);
        base += stride;
        if (base >= n) break;
        c.load(adv, base, n);
    }
}

// ---- separate merge launch (grids of more than kFusedMaxTiles tiles) ----

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
    const bool aligned = (reinterpret_cast<uintptr_t>(a.advantages) & 15u) == 0;
    if (plan.geo.num_tiles <= kFusedMaxTiles) {
        const int64_t blocks = std::min<int64_t>((N + kNormChunk - 1) / kNormChunk, kNormMaxBlocks);
        if (aligned)
            hipLaunchKernelGGL(normalize_fused_kernel<true>, dim3((unsigned)blocks),
                               dim3(kNormThreads), 0, s, a.advantages, N, tiles,
                               plan.geo.num_tiles, (double)eps, stats_out);
        else
            hipLaunchKernelGGL(normalize_fused_kernel<false>, dim3((unsigned)blocks),
                               dim3(kNormThreads), 0, s, a.advantages, N, tiles,
                               plan.geo.num_tiles, (double)eps, stats_out);
        return last_launch_status();
    }
    hipLaunchKernelGGL(stats_finalize_kernel, dim3(1), dim3(kStatThreads), 0, s, tiles,
                       plan.geo.num_tiles, (double)eps, result, stats_out);
    if ((st = last_launch_status()) != RLSCAN_OK) return st;
    const int64_t blocks = std::min<int64_t>((N + 1023) / 1024, (int64_t)1 << 20);
    hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.advantages, N,
                       result, aligned ? 1 : 0);
    return last_launch_status();
}

}  // namespace rlscan
