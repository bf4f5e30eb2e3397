// Permute: expert histogram, exclusive scan and stable scatter of the T*k
// token-expert assignments ("DeepSeek V3/R1 Inference Efficiency (2)",
// section 2.3.1, operator "Expert: prepare routed GEMM").
//
// Integer-only and deterministic.  Stability (ascending flat index inside
// each expert's segment) comes from ranking, never from atomics:
//   1. per-chunk histograms (LDS integer atomics; only counts, order-free);
//   2. one workgroup scans counts over experts and, per expert, over chunks:
//      offsets, counts, and the base position of every (chunk, expert);
//   3. each chunk ranks its items per expert with a wave64 multisplit
//      (ballots on the id bits give the mask of lanes holding the same
//      expert; rank = popcount of lower peers) plus the counts of the lower
//      waves of the chunk, and scatters src/dest.
// Sizes: chunk = 1024 items (16 waves); E <= 1024.
// Up to kSmallChunks chunks (a decode batch: T*k = 1024 at T = 128, k = 8)
// one workgroup does all three steps in one launch, taking the chunks in
// order with running per-expert bases: the same positions, without the two
// extra launches.
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kChunk = 1024;
constexpr int kChunkWaves = kChunk / kWave;
constexpr int kSmallChunks = 2;

static inline int nchunks(int R) { return (R + kChunk - 1) / kChunk; }

size_t permute_ws_bytes(int R, int E) {
    // chunk histograms / bases [nchunks][E] int32
    return (size_t)nchunks(R) * E * sizeof(int32_t) + 256;
}

__global__ __launch_bounds__(kChunk) void perm_hist_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                           int32_t* __restrict__ chunk_hist) {
    __shared__ int32_t cnt[1024];
    for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
    __syncthreads();
    const int f = blockIdx.x * kChunk + threadIdx.x;
    if (f < R) {
        const int e = ids[f];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // out-of-range ids are dropped
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kChunk) chunk_hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads turns chunk_hist [nch][E] into chunk_base in
// place and writes counts / offsets.  TPE threads share an expert (thread
// e*TPE + j owns the j-th contiguous run of chunks of expert e), so the chunk
// loops are nch / TPE long and their loads are independent.
template <int TPE>
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ chunk_hist, int nch, int E, int R,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
    __shared__ int32_t part[1024];     // per-thread partial sums (then their exclusive prefix)
    __shared__ int32_t tot[1024];      // per-expert totals (then exclusive prefix = offsets)
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x;
    const int e = tid / TPE, j = tid % TPE;
    const int run = (nch + TPE - 1) / TPE;
    const int c0 = min(j * run, nch), c1 = min(c0 + run, nch);
    int32_t sum = 0;
    if (e < E) {
#pragma unroll 8
        for (int c = c0; c < c1; ++c) sum += chunk_hist[(size_t)c * E + e];
    }
    part[tid] = sum;
    __syncthreads();
    if (j == 0) {
        int32_t acc = 0;
        for (int q = 0; q < TPE; ++q) {
            const int32_t v = part[tid + q];
            part[tid + q] = acc;
            acc += v;
        }
        tot[e] = e < E ? acc : 0;
    }
    __syncthreads();
    // exclusive scan of tot over experts (1024 entries, one per thread)
    const int lane = tid % kWave, w = tid / kWave;
    const int32_t c = tot[tid];
    int32_t v = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    if (lane == kWave - 1) wsum[w] = v;
    __syncthreads();
    int32_t wb = 0;
    for (int i = 0; i < w; ++i) wb += wsum[i];
    __syncthreads();
    tot[tid] = wb + v - c;            // exclusive prefix over experts
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = wb + v - c;
    }
    if (tid == 0) offsets[E] = R;
    __syncthreads();
    if (e < E) {
        int32_t base = tot[e] + part[tid];
#pragma unroll 8
        for (int cc = c0; cc < c1; ++cc) {
            const int32_t h = chunk_hist[(size_t)cc * E + e];
            chunk_hist[(size_t)cc * E + e] = base;
            base += h;
        }
    }
}

// Ranks of the items of one chunk (flat indices c0 .. c0+1023) within their
// expert: wave64 multisplit on the id bits; wcnt[w][e] receives the number
// of items of expert e in wave w.  Returns the rank among the wave's items of
// the same expert, or -1 for an item past R or with an out-of-range id.
__device__ __forceinline__ int chunk_rank(const int32_t* __restrict__ ids, int R, int E, int nbits, int c0,
                                          int32_t (*wcnt)[1024], int& e_out) {
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int f = c0 + tid;
    const int e0 = f < R ? ids[f] : -1;
    const bool valid = (unsigned)e0 < (unsigned)E;        // out-of-range ids are dropped
    const int e = valid ? e0 : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const uint64_t m = __ballot(valid && ((e >> b) & 1));
        peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int rank = __popcll(peers & lower);
    if (valid && (peers & lower) == 0) wcnt[w][e] = __popcll(peers);
    e_out = e;
    return valid ? rank : -1;
}

__global__ __launch_bounds__(kChunk) void perm_scatter_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                              int nbits, const int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ src, int32_t* __restrict__ dest) {
    __shared__ int32_t wcnt[kChunkWaves][1024];   // items of expert e in wave w
    const int tid = threadIdx.x, w = tid / kWave;
    const int f = blockIdx.x * kChunk + tid;
    // zero only the entries this chunk will read
    for (int i = tid; i < kChunkWaves * E; i += kChunk) wcnt[i / E][i % E] = 0;
    __syncthreads();
    int e;
    const int rank = chunk_rank(ids, R, E, nbits, blockIdx.x * kChunk, wcnt, e);
    __syncthreads();
    if (rank >= 0) {
        int pos = chunk_base[(size_t)blockIdx.x * E + e] + rank;
        for (int i = 0; i < w; ++i) pos += wcnt[i][e];
        src[pos] = f;
        dest[f] = pos;
    }
}

__global__ __launch_bounds__(kChunk) void perm_small_kernel(const int32_t* __restrict__ ids, int R, int E, int nbits,
                                                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ src, int32_t* __restrict__ dest) {
    __shared__ int32_t wcnt[kChunkWaves][1024];   // items of expert e in wave w of the current chunk
    __shared__ int32_t base[1024];                // per expert: count, then next free position
    __shared__ int32_t wsum[16];
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    base[tid] = 0;
    __syncthreads();
    for (int f = tid; f < R; f += kChunk) {
        const int e = ids[f];
        if ((unsigned)e < (unsigned)E) atomicAdd(&base[e], 1);   // counts only: order-free
    }
    __syncthreads();
    // exclusive scan over experts (1024 entries, one per thread; entries >= E are 0)
    const int32_t c = base[tid];
    int32_t v = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    if (lane == kWave - 1) wsum[w] = v;
    __syncthreads();
    int32_t wb = 0;
    for (int i = 0; i < w; ++i) wb += wsum[i];
    base[tid] = wb + v - c;
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = wb + v - c;
    }
    if (tid == 0) offsets[E] = R;
    for (int c0 = 0; c0 < R; c0 += kChunk) {
        for (int i = tid; i < kChunkWaves * E; i += kChunk) wcnt[i / E][i % E] = 0;
        __syncthreads();
        int e;
        const int rank = chunk_rank(ids, R, E, nbits, c0, wcnt, e);
        __syncthreads();
        if (rank >= 0) {
            int pos = base[e] + rank;
            for (int i = 0; i < w; ++i) pos += wcnt[i][e];
            src[pos] = c0 + tid;
            dest[c0 + tid] = pos;
        }
        __syncthreads();
        for (int e2 = tid; e2 < E; e2 += kChunk) {
            int32_t n = 0;
            for (int i = 0; i < kChunkWaves; ++i) n += wcnt[i][e2];
            base[e2] += n;
        }
        __syncthreads();   // the counts are read before the next chunk clears them
    }
}

hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* counts, int32_t* offsets,
                          int32_t* src, int32_t* dest, void* ws, hipStream_t s) {
    const int nch = nchunks(R);
    int32_t* chunk = (int32_t*)ws;
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    if (nch <= kSmallChunks) {
        hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(kChunk), 0, s, ids, R, E, nbits, counts, offsets, src,
                           dest);
        return hipGetLastError();
    }
    if (nch > 0) {
        hipLaunchKernelGGL(perm_hist_kernel, dim3(nch), dim3(kChunk), 0, s, ids, R, E, chunk);
    }
    // threads per expert: the largest power of two with E * TPE <= 1024
#define MOE_SCAN(TPEV) hipLaunchKernelGGL(perm_scan_kernel<TPEV>, dim3(1), dim3(1024), 0, s, chunk, nch, E, R, counts, offsets)
    if (E <= 8) MOE_SCAN(128);
    else if (E <= 16) MOE_SCAN(64);
    else if (E <= 32) MOE_SCAN(32);
    else if (E <= 64) MOE_SCAN(16);
    else if (E <= 128) MOE_SCAN(8);
    else if (E <= 256) MOE_SCAN(4);
    else if (E <= 512) MOE_SCAN(2);
    else MOE_SCAN(1);
#undef MOE_SCAN
    if (nch > 0) {
        hipLaunchKernelGGL(perm_scatter_kernel, dim3(nch), dim3(kChunk), 0, s, ids, R, E, nbits, chunk, src, dest);
    }
    return hipGetLastError();
}

}  // namespace moe
