// op_gae_norm.hip -- GAE with batch advantage normalisation (paper Sec. 9.3
// plans fused advantage normalisation; the formula is the usual whitening of
// PPO advantages):
//   adv_t = (A_t - mean) / (std + eps),  mean and unbiased std over all E*T steps.
// Batches whose tiles are all resident at once take a single launch instead
// (op_gae_norm_one.hip).  Otherwise two launches on the stream:
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

constexpr int kStatBatch = 4;  // triples a thread loads before adding them
// Grid sizes that take the statistics inside the normalising pass, by the
// workgroup size that pass uses: 256 threads up to 2048 tiles (each thread
// adds at most eight triples), 1024 threads up to 8192 tiles.  Larger grids
// merge the triples in a launch of their own.
constexpr int64_t kFusedSmallMaxTiles = 2048;
constexpr int64_t kFusedMaxTiles = 8192;
constexpr int kFinalThreads = 1024;

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

// Thread i's first batch: tiles i, i + THREADS, i + 2 THREADS, i + 3 THREADS.
template <int THREADS>
__device__ __forceinline__ void load_first_batch(const double* tiles, int64_t num_tiles,
                                                 StatD (&b)[kStatBatch]) {
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u)
        b[u] = load_triple(tiles, threadIdx.x + (int64_t)u * THREADS, num_tiles);
}

// Workgroup totals of x[0..K) over its THREADS threads; every thread gets
// them.  The wave sums (wave_sum_f64, scan_kernel.hpp) are added in wave
// order: the same bits on every call.
template <int THREADS, int K>
__device__ __forceinline__ void block_sum(double (&x)[K], double (&sh)[K][THREADS / 64]) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] = wave_sum_f64(x[k]);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int k = 0; k < K; ++k) sh[k][w] = x[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        x[k] = 0.0;
#pragma unroll
        for (int v = 0; v < THREADS / 64; ++v) x[k] += sh[k][v];
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
template <int THREADS>
__device__ BatchStats batch_stats(const double* tiles, int64_t num_tiles,
                                  const StatD (&first)[kStatBatch],
                                  double (&sh)[2][THREADS / 64]) {
    const int64_t step = (int64_t)kStatBatch * THREADS;
    double ns[2] = {0.0, 0.0};  // count, sum of n m
#pragma unroll
    for (int u = 0; u < kStatBatch; ++u) {
        ns[0] += first[u].n;
        ns[1] = fma(first[u].n, first[u].m, ns[1]);
    }
    for (int64_t t0 = threadIdx.x + step; t0 < num_tiles; t0 += step) {
        StatD b[kStatBatch];
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) b[u] = load_triple(tiles, t0 + u * THREADS, num_tiles);
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) {
            ns[0] += b[u].n;
            ns[1] = fma(b[u].n, b[u].m, ns[1]);
        }
    }
    block_sum<THREADS, 2>(ns, sh);
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
        for (int u = 0; u < kStatBatch; ++u) b[u] = load_triple(tiles, t0 + u * THREADS, num_tiles);
#pragma unroll
        for (int u = 0; u < kStatBatch; ++u) {
            const double d = b[u].m - mean;
            q[0] += fma(b[u].n * d, d, b[u].m2);
        }
    }
    double (&sh1)[1][THREADS / 64] = *reinterpret_cast<double (*)[1][THREADS / 64]>(&sh[0][0]);
    block_sum<THREADS, 1>(q, sh1);
    return BatchStats{mean, ns[0] > 1.0 ? sqrt(q[0] / (ns[0] - 1.0)) : 0.0};
}

// One workgroup of kFinalThreads threads.  result[0] = mean, result[1] = std,
// result[2] = 1 / (std + eps).
__global__ __launch_bounds__(kFinalThreads) void stats_finalize_kernel(const double* tiles,
                                                                      int64_t num_tiles,
                                                                      double eps, double* result,
                                                                      double* user) {
    __shared__ double sh[2][kFinalThreads / 64];
    StatD first[kStatBatch];
    load_first_batch<kFinalThreads>(tiles, num_tiles, first);
    const BatchStats st = batch_stats<kFinalThreads>(tiles, num_tiles, first, sh);
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
constexpr int kNormVecs = 4;  // groups of four advantages per thread and chunk
constexpr int64_t kNormMaxThreadsTotal = 256 * 1024;  // workgroups x threads at most

// A thread's sixteen advantages of one chunk: group k is the four consecutive
// steps at base + 4 (k * THREADS + thread) when VEC (16-byte accesses), else
// element k * THREADS + thread for k < 16.
template <int THREADS, bool VEC>
struct NormChunk {
    static constexpr int64_t kChunkMax = (int64_t)THREADS * kNormVecs * 4;
    float v[kNormVecs * 4];

    __device__ __forceinline__ int64_t index(int64_t base, int k, int c) const {
        return VEC ? base + ((int64_t)k * THREADS + threadIdx.x) * 4 + c
                   : base + (int64_t)(4 * k + c) * THREADS + threadIdx.x;
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
                // with device scope, over the chunk (see store16): 27.9-28.0 ->
                // 26.5-26.9 us per normalised 4096 x 1024 call
                const int64_t left = n - base;
                const uint32_t extent = (uint32_t)(left < kChunkMax ? left : kChunkMax) * 4u;
                store16<true>(adv + base, (uint32_t)(i - base) * 4u, extent, x);
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
template <int THREADS, bool VEC>
__global__ __launch_bounds__(THREADS) void normalize_fused_kernel(
    float* adv, int64_t n, const double* tiles, int64_t num_tiles, double eps, double* user) {
    constexpr int64_t kChunk = (int64_t)THREADS * kNormVecs * 4;
    __shared__ double sh[2][THREADS / 64];
    StatD first[kStatBatch];
    load_first_batch<THREADS>(tiles, num_tiles, first);
    int64_t base = (int64_t)blockIdx.x * kChunk;
    NormChunk<THREADS, VEC> c;
    c.load(adv, base, n);
    const BatchStats st = batch_stats<THREADS>(tiles, num_tiles, first, sh);
    if (user && blockIdx.x == 0 && threadIdx.x == 0) {
        user[0] = st.mean;
        user[1] = st.sd;
    }
    const float mean = (float)st.mean;
    const float inv = (float)(1.0 / (st.sd + eps));
    const int64_t stride = (int64_t)gridDim.x * kChunk;
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

template <int THREADS>
rlscan_status launch_fused(float* adv, int64_t N, const double* tiles, int64_t num_tiles, float eps,
                           double* stats_out, bool aligned, hipStream_t s) {
    constexpr int64_t chunk = (int64_t)THREADS * kNormVecs * 4;
    const int64_t blocks = std::min<int64_t>((N + chunk - 1) / chunk, kNormMaxThreadsTotal / THREADS);
    if (aligned)
        hipLaunchKernelGGL((normalize_fused_kernel<THREADS, true>), dim3((unsigned)blocks),
                           dim3(THREADS), 0, s, adv, N, tiles, num_tiles, (double)eps, stats_out);
    else
        hipLaunchKernelGGL((normalize_fused_kernel<THREADS, false>), dim3((unsigned)blocks),
                           dim3(THREADS), 0, s, adv, N, tiles, num_tiles, (double)eps, stats_out);
    return last_launch_status();
}

}  // namespace

rlscan_status launch_gae_norm(const GaeArgs& args, const Plan& plan, void* ws, size_t stats_off,
                              size_t words_off, bool single_ok, int64_t N, float eps,
                              double* stats_out, hipStream_t s) {
    GaeArgs a = args;
    rlscan_status st;
    if (single_ok) {
        a.norm_words = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + words_off);
        a.eps = eps;
        a.user_stats = stats_out;
        bool launched = false;
        st = launch_gae_norm_one(a, plan, ws, s, launched);
        if (st != RLSCAN_OK || launched) return st;
    }
    double* tiles = reinterpret_cast<double*>(static_cast<uint8_t*>(ws) + stats_off);
    double* result = tiles + 4 * plan.geo.num_tiles;
    a.tile_stats = tiles;
    if (!a.truncateds)
        st = launch_gae_op<kStatsOut>(a, plan, ws, s);
    else if (!a.bootstrap_values)
        st = launch_gae_op<kStatsOut | kTrunc>(a, plan, ws, s);
    else
        st = launch_gae_op<kStatsOut | kTrunc | kBoot2D>(a, plan, ws, s);
    if (st != RLSCAN_OK) return st;
    const bool aligned = (reinterpret_cast<uintptr_t>(a.advantages) & 15u) == 0;
    if (plan.geo.num_tiles <= kFusedSmallMaxTiles)
        return launch_fused<256>(a.advantages, N, tiles, plan.geo.num_tiles, eps, stats_out, aligned, s);
    if (plan.geo.num_tiles <= kFusedMaxTiles)
        return launch_fused<1024>(a.advantages, N, tiles, plan.geo.num_tiles, eps, stats_out, aligned, s);
    hipLaunchKernelGGL(stats_finalize_kernel, dim3(1), dim3(kFinalThreads), 0, s, tiles,
                       plan.geo.num_tiles, (double)eps, result, stats_out);
    if ((st = last_launch_status()) != RLSCAN_OK) return st;
    const int64_t blocks = std::min<int64_t>((N + 1023) / 1024, (int64_t)1 << 20);
    hipLaunchKernelGGL(normalize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.advantages, N,
                       result, aligned ? 1 : 0);
    return last_launch_status();
}

}  // namespace rlscan
