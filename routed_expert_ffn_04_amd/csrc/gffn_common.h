// Shared definitions of the grouped expert FFN kernels: arguments, MFMA
// operand traits, group lookup, and the persistent work queues.
#pragma once
#include <atomic>

#include "common.h"
#include "internal.h"

namespace moe {

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2, DT_MXFP4 = 3 };   // weight types (MXFP4: MXFP8 activations)

template <int DT> struct Op;
template <> struct Op<DT_F32> {
    static constexpr int EB = 4;      // bytes per element
    static constexpr int KI = 4;      // k per MFMA
    static constexpr int LB = 4;      // bytes per lane per MFMA operand
    __device__ static f32x4 mma(const uint8_t* a, const uint8_t* b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(*(const float*)a, *(const float*)b, c, 0, 0, 0);
    }
};
template <> struct Op<DT_BF16> {
    static constexpr int EB = 2, KI = 32, LB = 16;
    __device__ static f32x4 mma(const uint8_t* a, const uint8_t* b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)a, *(const bf16x8*)b, c, 0, 0, 0);
    }
};
template <> struct Op<DT_E4M3> {
    static constexpr int EB = 1, KI = 128, LB = 32;
    __device__ static f32x4 mma(const uint8_t* a, const uint8_t* b, f32x4 c) {
        const i32x4 a0 = *(const i32x4*)a, a1 = *(const i32x4*)(a + 16);
        const i32x4 b0 = *(const i32x4*)b, b1 = *(const i32x4*)(b + 16);
        const i32x8 av = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const i32x8 bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        // operand formats 0/0 = FP8 E4M3; e8m0 scales 127 = 1.0
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
    }
};

constexpr int kXcds = 8;          // MI355X: 8 accelerator dies, each with its own L2
constexpr int kClasses = 3;       // tile classes by rows per group

// A work list of m-tiles (group, first row) for one tile class, written by
// the list builder; the tiles of a launch are (entry, n-tile) pairs.
struct TileList {
    const int2* entries;
    const int* count;           // number of entries
};

struct GArgs {
    // activation scales: fp32 [rows][H/128] (E4M3), or E8M0 bytes [rows][H/32] (MXFP8)
    const uint8_t* a; const float* a_scale; const int32_t* src; int src_div;
    const uint8_t* a_sh; const float* a_sh_scale;
    const int32_t* offsets; int G; int R_max; int S;
    Bank routed, shared;
    int H, I;
    uint8_t* h; float* h_scale;        // [R_max + S][I], [R_max + S][I/128] (MXFP4: E8M0 bytes [..][I/32])
    void* y; void* y_sh; int y_bf16;   // routed outputs bf16 (else fp32 unless y_e4m3)
    int y_e4m3; float* y_scale;        // routed outputs as e4m3 + [R_max][H/128] scales (large fp8 tiles)
    int y_sh_bf16;                     // shared outputs bf16 (else fp32)
};

struct GroupInfo {
    int p0, m, e, shared;
};

__device__ __forceinline__ GroupInfo group_info(const GArgs& A, int g) {
    GroupInfo gi;
    if (g < A.G) {
        gi.p0 = min(max(A.offsets[g], 0), A.R_max);
        gi.m = min(max(A.offsets[g + 1] - gi.p0, 0), A.R_max - gi.p0);
        gi.e = g;
        gi.shared = 0;
    } else {
        gi.p0 = 0;
        gi.m = A.S;
        gi.e = 0;
        gi.shared = 1;
    }
    return gi;
}

// Row index of tile row r in the h buffer (routed rows first, then shared).
__device__ __forceinline__ int h_row(const GArgs& A, const GroupInfo& gi, int r) {
    return gi.shared ? A.R_max + r : gi.p0 + r;
}

// silu(g) * u with a hardware reciprocal (about 1 ulp) in place of the
// divide; exp(-g) overflowing to +inf gives the exact limit 0.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Static, die-aware assignment of the tiles of a list to a persistent grid.
// Workgroups are dispatched to the kXcds dies round robin, so workgroup b runs
// on die b % kXcds.  The tile range is cut into kXcds contiguous chunks and
// the workgroups of die x stride through chunk x: consecutive tiles (the
// n-tiles of one m-tile, which share activation rows) stay in one die's L2.
// No atomics: every tile costs about the same within a class, and the list is
// already in longest-first order.  Iterate with
//   for (TileIter it(L, per_entry); it.valid(); it.next()) { ... it.t ... }
struct TileIter {
    long t, end, stride;
    __device__ TileIter(const TileList& L, int per_entry) {
        const long total = (long)(*L.count) * per_entry;
        const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
        const int nwg_x = ((int)gridDim.x - x + kXcds - 1) / kXcds;
        const long lo = total * x / kXcds;
        end = total * (x + 1) / kXcds;
        t = lo + j;
        stride = nwg_x;
    }
    __device__ bool valid() const { return t < end; }
    __device__ void next() { t += stride; }
};

// Tile t of a list -> (entry, n-tile).  Entry-major order keeps the n-tiles
// of one m-tile together (one die's L2 serves their shared activation rows);
// n-major order keeps the m-tiles of one weight tile together, so a group cut
// into several 16-row m-tiles reads each weight tile from HBM once and from
// L2 for the other m-tiles.
template <bool NMAJOR>
__device__ __forceinline__ int2 tile_coords(const TileList& L, long t, int ntn) {
    if (NMAJOR) {
        const int c = *L.count;
        return make_int2((int)(t % c), (int)(t / c));
    }
    return make_int2((int)(t / ntn), (int)(t % ntn));
}

// s_waitcnt with only the vector-memory count: vmcnt(n), expcnt and
// lgkmcnt left at their maxima (gfx9 encoding: vmcnt[3:0] | expcnt << 4 |
// lgkmcnt << 8 | vmcnt[5:4] << 14).  The hardware barrier itself does not wait
// for a wave's direct global->LDS loads; __syncthreads does, because the
// compiler puts vmcnt(0) in front of its release fence (direct loads count as
// LDS writes), so wait_vm<0>() before it only states the need.  A barrier
// that must leave some loads in flight is an s_barrier after an explicit
// count.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Host launchers of the kernel families (gffn_tile.hip, gffn_stream.hip, gffn_mid.hip, gffn_big.hip,
// gffn_mx.hip, gffn_mxbig.hip).
hipError_t launch_tile_gateup(int dt, const GArgs& A, const TileList& L, int bm, hipStream_t s);
hipError_t launch_tile_down(int dt, const GArgs& A, const TileList& L, int bm, hipStream_t s);
hipError_t launch_stream_gateup(int mb, const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_stream_down(int mb, const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_mid_gateup(const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_mid_down(const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_big_gateup(int dt, const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_big_down(int dt, const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_mx_gateup(int mb, const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_mx_down(int mb, const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_mxbig_gateup(const GArgs& A, const TileList& L, hipStream_t s);
hipError_t launch_mxbig_down(const GArgs& A, const TileList& L, hipStream_t s);
int device_cu_count();

// Launch constants (persistent grid sizes) cached per device: computed on the
// first launch on each device with that device current.  Concurrent first
// calls compute the same value, so publishing it through a relaxed atomic is
// race-free; devices beyond kMaxDevices recompute every time.
constexpr int kMaxDevices = 64;
using DeviceCache = std::atomic<int>[kMaxDevices];

template <class F>
int per_device(DeviceCache& cache, F compute) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return compute();
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        v = compute();
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

}  // namespace moe
