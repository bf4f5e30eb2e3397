// Grouped expert FFN: scheduling and host launch ("DeepSeek V3/R1 Inference
// Efficiency (2)", section 1.b: grouped-GEMM efficiency depends on the number
// of groups and the rows per group; section 2.3.1 / 2.4.1: the routed and
// shared expert GEMMs at prefill and decode sizes).
//
// Every group (routed expert g, plus the shared expert as group G) is put in
// one of three tile classes by its row count m, read on the device:
//   class 0: m <= 16          weight-streaming tiles of 16 rows (bf16
//                             where the large tiles do not apply)
//   class 1: 16 < m <= 256    64 x 256 MFMA tiles with a three-stage load
//                             ring (gffn_mid.hip; bf16 where the large tiles
//                             apply, then for 0 < m <= 256), else
//                             weight-streaming tiles of 64 rows
//   class 2: otherwise        256 x 256 MFMA tiles (bf16 / e4m3, gffn_big.hip),
//                             or 64-row LDS tiles (fp32 or H % 256 != 0)
// (fp32 and e4m3 layers put every group in class 2; MXFP4 layers use the
// MX weight-streaming tiles of gffn_mx.hip, 16 rows for m <= 32, and the
// 256 x 256 MX tiles of gffn_mxbig.hip above; groups of 33-256 rows join the
// 16-row tiles when there are at most four of them, else the large tiles,
// and take 64-row streaming tiles only where the large tiles do not apply).  One single-workgroup kernel
// writes, per class, the list of (group, first row) m-tiles with the heaviest
// groups first (longest-processing-time order); then each class's gate/up
// kernel and down kernel run as persistent grids that walk their list (see
// TileIter).  Nothing is copied to the host, so the whole call is
// asynchronous.
#include "gffn_common.h"

#include <algorithm>

namespace moe {

struct ClassSpec {
    int mlo[kClasses], mhi[kClasses], bm[kClasses];
    // Class 1 (weight-streaming tiles of 64 rows re-read the group's rows once
    // per 32 output columns) moves into class 2 (256-row tiles) when it has at
    // least this many members: then there are enough groups to fill the chip
    // with the large tiles, which read every row once per 128/256 columns.
    // 0: never.
    int promote_min;
    // Class 1 moves into class 0 (16-row tiles, weight tiles shared through
    // L2 by the m-tiles of a group) when it has 1 .. demote_max members: a
    // handful of groups (the shared expert at decode) would otherwise run
    // alone in a launch that fills a fraction of the chip.  0: never.
    int demote_max;
    // Class 1 runs the 64-row tiles with a three-stage load ring
    // (gffn_mid.hip) instead of the weight-streaming tiles.
    int mid1;
};

struct ListsOut {
    int2* entries[kClasses];
    int maxe[kClasses];
    int* counts;      // [kClasses]
};

constexpr int kMaxGroups = 1025;   // 1024 routed + shared
constexpr int kSortSlots = 2048;   // power of two >= kMaxGroups; one compare per thread and pass

// Exclusive scan of arr[0 .. n) in place by a 1024-thread workgroup (chunks of
// 1024 with a running carry); returns the total.  Every thread must call it.
__device__ int block_scan_exclusive(int* arr, int n, int* wsum) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    int carry = 0;
    for (int base = 0; base < n; base += 1024) {
        const int i = base + (int)threadIdx.x;
        const int v = i < n ? arr[i] : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(x, d, kWave);
            if (lane >= d) x += o;
        }
        if (lane == kWave - 1) wsum[w] = x;
        __syncthreads();
        int wb = 0, tot = 0;
        for (int k = 0; k < 16; ++k) {
            wb += k < w ? wsum[k] : 0;
            tot += wsum[k];
        }
        if (i < n) arr[i] = carry + wb + x - v;
        __syncthreads();
        carry += tot;
    }
    return carry;
}

// One workgroup of 1024 threads.  Group g's rank inside its class is the
// number of class members with more rows (or as many rows and a lower
// index); each class's m-tiles are laid out in rank order, so the heaviest
// groups come first.  The ranks come from one bitonic sort of the keys
// (class, rows descending, group) over 2048 slots in LDS.
__global__ __launch_bounds__(1024) void gffn_build_lists(const int32_t* __restrict__ offsets, int G, int S,
                                                         int R_max, ClassSpec cs, ListsOut out) {
    __shared__ int m_of[kMaxGroups];
    __shared__ int cls_of[kMaxGroups];
    __shared__ unsigned long long keys[kSortSlots];   // class << 42 | (2^31 - 1 - m) << 11 | g; unused: ~0
    __shared__ int rank_of[kMaxGroups];
    __shared__ int nt_by_rank[kClasses][kMaxGroups];
    __shared__ int members[kClasses];
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    const int ng = min(G + (S > 0 ? 1 : 0), kMaxGroups);
    if (tid < kClasses) members[tid] = 0;
    __syncthreads();
    for (int g = tid; g < ng; g += 1024) {
        int m;
        if (g < G) {
            const int p0 = min(max(offsets[g], 0), R_max);
            m = min(max(offsets[g + 1] - p0, 0), R_max - p0);
        } else {
            m = S;
        }
        int c = -1;
        for (int k = 0; k < kClasses; ++k)
            if (m > cs.mlo[k] && m <= cs.mhi[k]) { c = k; break; }
        c = m > 0 ? c : -1;
        m_of[g] = m;
        cls_of[g] = c;
        if (c >= 0) atomicAdd(&members[c], 1);
    }
    __syncthreads();
    const int m1 = members[1];
    const int to = (cs.demote_max > 0 && m1 > 0 && m1 <= cs.demote_max) ? 0
                 : (cs.promote_min > 0 && m1 >= cs.promote_min)        ? 2 : 1;
    if (to != 1) {
        for (int g = tid; g < ng; g += 1024)
            if (cls_of[g] == 1) cls_of[g] = to;
        __syncthreads();
        if (tid == 0) {
            members[to] += m1;
            members[1] = 0;
        }
        __syncthreads();
    }
    for (int i = tid; i < kSortSlots; i += 1024) {
        const int c = i < ng ? cls_of[i] : -1;
        keys[i] = c < 0 ? ~0ull
                        : ((unsigned long long)c << 42) | ((unsigned long long)(0x7fffffff - m_of[i]) << 11) |
                              (unsigned long long)i;
    }
    __syncthreads();
    // ascending bitonic sort of the first n2 slots (the smallest power of two
    // >= ng; the slots past ng hold ~0 and stay last): thread t < n2/2
    // compares slot i (bit j of i clear) with i + j
    int n2 = 2;
    while (n2 < ng) n2 <<= 1;
    for (int k = 2; k <= n2; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (tid < n2 / 2) {
                const int i = ((tid & ~(j - 1)) << 1) | (tid & (j - 1));
                const unsigned long long a = keys[i], b = keys[i + j];
                if ((a > b) == ((i & k) == 0)) {
                    keys[i] = b;
                    keys[i + j] = a;
                }
            }
            __syncthreads();
        }
    // a class's members are contiguous in the sorted order, heaviest first
    for (int i = tid; i < kSortSlots; i += 1024) {
        const unsigned long long key = keys[i];
        if (key == ~0ull) continue;
        const int c = (int)(key >> 42), g = (int)(key & 2047);
        int first = 0;
        for (int q = 0; q < c; ++q) first += members[q];
        const int rank = i - first;
        nt_by_rank[c][rank] = (m_of[g] + cs.bm[c] - 1) / cs.bm[c];
        rank_of[g] = rank;
    }
    __syncthreads();
    for (int c = 0; c < kClasses; ++c) {
        const int total = block_scan_exclusive(nt_by_rank[c], members[c], wsum);
        if (tid == 0) out.counts[c] = min(total, out.maxe[c]);
    }
    __syncthreads();
    for (int g = tid; g < ng; g += 1024) {
        const int c = cls_of[g];
        if (c < 0) continue;
        const int base = nt_by_rank[c][rank_of[g]];
        const int nt = (m_of[g] + cs.bm[c] - 1) / cs.bm[c];
        for (int i = 0; i < nt && base + i < out.maxe[c]; ++i) out.entries[c][base + i] = make_int2(g, i * cs.bm[c]);
    }
}

int device_cu_count() {
    static DeviceCache cache;
    return per_device(cache, [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    });
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Large groups use the 256 x 256 tiles of gffn_big.hip (bf16 / e4m3 with
// H a multiple of 256, row offsets of the activation, h and per-expert weight
// matrices within 32 bits), otherwise the 64-row LDS tiles of gffn_tile.hip.
static bool use_big(int dt, int H, int I, int R_max, int S) {
    if (!(dt == DT_BF16 || dt == DT_E4M3) || H % 256 != 0) return false;
    const uint64_t eb = dt == DT_BF16 ? 2 : 1, lim = (uint64_t)1 << 32;
    return (uint64_t)std::max(R_max, S) * H * eb < lim && ((uint64_t)R_max + S) * I * eb < lim &&
           (uint64_t)H * I * eb < lim;
}

bool gffn_e4m3_y_supported(int H, int I, int R_max, int S) { return use_big(DT_E4M3, H, I, R_max, S); }

// Large MXFP4 tiles (gffn_mxbig.hip): 256-column down tiles, 32-bit byte
// offsets of activation / h rows and of a weight matrix.
static bool use_mxbig(int H, int I, int R_max, int S) {
    const uint64_t lim = (uint64_t)1 << 32;
    return H % 256 == 0 && (uint64_t)std::max(R_max, S) * H < lim && ((uint64_t)R_max + S) * I < lim &&
           (uint64_t)H * I / 2 < lim;
}

constexpr int kDemoteMax = 4;

// MXFP4: groups of up to this many rows take the 16-row streaming tiles
// (several m-tiles of one group re-read its weights, mostly from L2).  With
// 256 groups, 24 and 32 rows ran 16% and 13% faster there than on the
// 256 x 256 MX tiles; 48 and 64 rows 24% and 60% slower.
constexpr int kMxC0Max = 32;

static ClassSpec class_spec(int dt, int H, int I, int R_max, int S) {
    ClassSpec c{};
    const int bm2 = use_big(dt, H, I, R_max, S) ? 256 : 64;
    if (dt == DT_MXFP4) {
        const bool big = use_mxbig(H, I, R_max, S);
        c.mlo[0] = 0;  c.mhi[0] = kMxC0Max; c.bm[0] = 16;
        c.mlo[1] = kMxC0Max; c.mhi[1] = big ? 256 : 1 << 30;  c.bm[1] = 64;
        c.mlo[2] = 256; c.mhi[2] = big ? 1 << 30 : 0;  c.bm[2] = 256;
        c.demote_max = kDemoteMax;
        // with the large MX tiles, the middle class never keeps its groups: up
        // to kDemoteMax of them join the 16-row tiles, more join the large
        // tiles (16 groups of 65-256 rows: 2-3x faster there than on the
        // 64-row streaming tiles), so its launches are skipped
        c.promote_min = big ? kDemoteMax + 1 : 0;
    } else if (dt == DT_BF16) {
        // with the large tiles available (H % 256 == 0, 32-bit offsets), every
        // group of up to 256 rows takes the 64-row ring tiles, which share
        // those limits (also the few-row groups of a decode batch: 6% faster
        // there than the 16-row weight-streaming tiles)
        c.mlo[0] = 0;  c.mhi[0] = bm2 == 256 ? 0 : 16;       c.bm[0] = 16;
        c.mlo[1] = bm2 == 256 ? 0 : 16; c.mhi[1] = 256;      c.bm[1] = 64;
        c.mlo[2] = 256; c.mhi[2] = 1 << 30; c.bm[2] = bm2;
        c.mid1 = bm2 == 256;
        c.demote_max = bm2 == 256 ? 0 : kDemoteMax;
    } else {
        c.mlo[0] = 0;  c.mhi[0] = 0;        c.bm[0] = 16;   // unused
        c.mlo[1] = 0;  c.mhi[1] = 0;        c.bm[1] = 64;   // unused
        c.mlo[2] = 0;  c.mhi[2] = 1 << 30;  c.bm[2] = bm2;
    }
    return c;
}

// Upper bound of the entries of each class (host-side, from R_max, G, S).
static void max_entries(int R_max, int G, int S, const ClassSpec& c, int out[kClasses]) {
    const long rows = (long)R_max + S;
    const long groups = (long)G + (S > 0 ? 1 : 0);
    for (int k = 0; k < kClasses; ++k) {
        if (c.mhi[k] <= c.mlo[k]) { out[k] = 0; continue; }
        // each member group has m > mlo, so at most rows / (mlo+1) of them
        // (class 2 may also receive class 1's groups)
        const int lo = (k == 2 && c.promote_min > 0) ? c.mlo[1] : c.mlo[k];
        const long members = std::min(groups, rows / (lo + 1));
        out[k] = (int)std::min<long>(rows / c.bm[k] + members, 1L << 30);
    }
}

size_t gffn_ws_bytes(int R_max, int G, int S, int H, int I, int dt) {
    const size_t rows = (size_t)R_max + S;
    const int eb = dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : 1;
    const ClassSpec cs = class_spec(dt, H, I, R_max, S);
    int me[kClasses];
    max_entries(R_max, G, S, cs, me);
    size_t b = align256(rows * I * eb);
    b += align256(rows * (I / 128) * sizeof(float));
    for (int k = 0; k < kClasses; ++k) b += align256((size_t)std::max(me[k], 1) * sizeof(int2));
    b += align256(sizeof(int) * kClasses);
    return b;
}

hipError_t launch_gffn(const GffnProblem& p, void* ws, hipStream_t s) {
    GArgs A;
    A.a = (const uint8_t*)p.a; A.a_scale = p.a_scale; A.src = p.src; A.src_div = p.src_div;
    A.a_sh = (const uint8_t*)p.a_sh; A.a_sh_scale = p.a_sh_scale;
    A.offsets = p.offsets; A.G = p.G; A.R_max = p.R_max; A.S = p.has_shared ? p.S : 0;
    A.routed = p.routed; A.shared = p.shared; A.H = p.H; A.I = p.I;
    A.y = p.y; A.y_sh = p.y_sh; A.y_bf16 = p.y_bf16;
    A.y_e4m3 = p.y_e4m3; A.y_scale = p.y_scale; A.y_sh_bf16 = p.y_sh_bf16;
    const size_t rows = (size_t)p.R_max + A.S;
    const int eb = p.dt == DT_F32 ? 4 : p.dt == DT_BF16 ? 2 : 1;
    const ClassSpec cs = class_spec(p.dt, p.H, p.I, p.R_max, A.S);
    int me[kClasses];
    max_entries(p.R_max, p.G, A.S, cs, me);

    uint8_t* w = (uint8_t*)ws;
    A.h = w; w += align256(rows * p.I * eb);
    A.h_scale = (float*)w; w += align256(rows * (p.I / 128) * sizeof(float));
    ListsOut lo;
    for (int k = 0; k < kClasses; ++k) {
        lo.entries[k] = (int2*)w;
        lo.maxe[k] = me[k];
        w += align256((size_t)std::max(me[k], 1) * sizeof(int2));
    }
    lo.counts = (int*)w;

    hipLaunchKernelGGL(gffn_build_lists, dim3(1), dim3(1024), 0, s, p.offsets, p.G, A.S, p.R_max, cs, lo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    TileList up[kClasses], dn[kClasses];
    for (int k = 0; k < kClasses; ++k) {
        up[k] = TileList{lo.entries[k], lo.counts + k};
        dn[k] = TileList{lo.entries[k], lo.counts + k};
    }
    // phase 1 (all classes), then phase 2: a group's down tiles need all of its h
    // the middle class always moves its groups out (demoted or promoted)
    const bool c1_empty = cs.promote_min > 0 && cs.promote_min == cs.demote_max + 1;
    // classes no group can reach under the caller's row bound are not launched
    // (their lists stay empty: a group lands only in a class whose range or
    // whose promotion source range it reaches)
    bool reach[kClasses];
    for (int k = 0; k < kClasses; ++k) {
        const bool own = p.m_max <= 0 || p.m_max > cs.mlo[k];
        const bool promoted = k == 2 && cs.promote_min > 0 && (p.m_max <= 0 || p.m_max > cs.mlo[1]);
        reach[k] = own || promoted;
    }
    for (int k = 0; k < kClasses && e == hipSuccess; ++k) {
        if (me[k] == 0 || (k == 1 && c1_empty) || !reach[k]) continue;
        e = p.dt == DT_MXFP4 ? (k == 2 ? launch_mxbig_gateup(A, up[k], s) : launch_mx_gateup(k == 0 ? 1 : 4, A, up[k], s))
          : k == 1 && cs.mid1 ? launch_mid_gateup(A, up[k], s)
          : k < 2 ? launch_stream_gateup(k == 0 ? 1 : 4, A, up[k], s)
                  : cs.bm[k] == 256 ? launch_big_gateup(p.dt, A, up[k], s) : launch_tile_gateup(p.dt, A, up[k], cs.bm[k], s);
    }
    for (int k = 0; k < kClasses && e == hipSuccess; ++k) {
        if (me[k] == 0 || (k == 1 && c1_empty) || !reach[k]) continue;
        e = p.dt == DT_MXFP4 ? (k == 2 ? launch_mxbig_down(A, dn[k], s) : launch_mx_down(k == 0 ? 1 : 4, A, dn[k], s))
          : k == 1 && cs.mid1 ? launch_mid_down(A, dn[k], s)
          : k < 2 ? launch_stream_down(k == 0 ? 1 : 4, A, dn[k], s)
                  : cs.bm[k] == 256 ? launch_big_down(p.dt, A, dn[k], s) : launch_tile_down(p.dt, A, dn[k], cs.bm[k], s);
    }
    return e;
}

}  // namespace moe
