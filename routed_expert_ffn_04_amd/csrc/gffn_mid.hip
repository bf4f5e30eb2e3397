// Grouped expert FFN, 64-row tiles for bf16 groups of up to 256 rows.
//
// "DeepSeek V3/R1 Inference Efficiency (2)", section 1.b: grouped-GEMM
// efficiency depends on the rows per group.  A group of a few dozen rows (or,
// in a decode batch, a few) multiplies a full [H, 2I] and [I, H] weight pair,
// so its cost is streaming those weights; the 256-row tiles of gffn_big.hip
// spend most of each stage's loads on padding rows and keep only one 32 KiB
// weight stage in flight.
//
// Tile: 64 rows x 256 MFMA columns (gate/up: 128 gate + 128 up columns of the
// same 128 h columns; down: 256 output columns), K staged 128 bytes (64 bf16)
// at a time through a three-deep LDS ring (40 KiB a stage: 64 activation rows
// then 256 weight rows) fed by direct global->LDS 16-byte loads, so two
// stages (64 KiB of weights) are in flight while one is computed.  The rows
// are XOR-swizzled as in the large tiles.
// 8 waves (2 along M x 4 along N), each computing 32 x 64 with
// v_mfma_f32_32x32x16_bf16, two per k-step (gate/up: the gate and the up
// block of the same 32 h columns, so SwiGLU needs no exchange).
// The m-tiles of a group that share a weight tile are adjacent in the tile
// order (n-tile-major, m-tiles innermost), so a weight tile is read from HBM
// once per die.
#include "gffn_common.h"

namespace moe {
namespace {

constexpr int kM = 64;                        // rows per tile
constexpr int kN = 256;                       // MFMA columns per tile
constexpr int kStage = 128;                   // K bytes per stage
constexpr int kRows = kM + kN;                // LDS rows per stage
constexpr int kStageBytes = kRows * kStage;   // 40 KiB
constexpr int kRing = 3;                      // stages in the ring
constexpr int kLoads = kRows * 8 / kWave / 8; // direct loads per wave and stage (16 B per lane)
static_assert(kLoads * kWave * 8 == kRows * 8, "loads cover the stage");

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kStage + ((chunk ^ swz_key(row)) << 4); }

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// 16-byte bf16 fragment (32x32x16 operand) of k-step ks: row, bytes [32 ks + 16 (lane/32), +16)
__device__ __forceinline__ bf16x8 frag16(const uint8_t* base, int row, int lane, int ks) {
    return *(const bf16x8*)(base + swz(row, ks * 2 + lane / 32));
}

// Workgroup barrier once this wave's LDS operations have completed and at
// most N of its vector-memory operations are outstanding (loads complete in
// issue order).  __syncthreads would wait for every direct load in flight,
// the next stage's included.
template <int N>
__device__ __forceinline__ void barrier_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The direct loads of a stage: instruction q of wave w fills LDS rows
// 8 (kLoads w + q) .. +7 (lane l: row + l/8, position l%8), all from one
// matrix (activation rows below kM, weight rows above), so each
// instruction's base address is wave-uniform.  off: the lane's byte offsets
// from those bases, the same for every stage of a tile.
struct Loads {
    const uint8_t* base[kLoads];
    uint32_t off[kLoads];
};

__device__ __forceinline__ void issue_stage(uint8_t* buf, const Loads& ld, int s, int wave) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(ld.base[q] + ld.off[q] + (uint32_t)s * kStage),
                                         (lds_void*)(buf + (kLoads * wave + q) * 1024), 16, 0, 0);
}

}  // namespace

// PHASE 0: gate/up (+SwiGLU epilogue, bf16 h); PHASE 1: down.
template <int PHASE>
__global__ __launch_bounds__(512) void mid_kernel(GArgs A, TileList L) {
    const int H = A.H, I = A.I;
    const int KB = (PHASE == 0 ? H : I) * 2;           // bytes per row of the reduction
    const int NOUT = PHASE == 0 ? I : H;
    const int ncol = PHASE == 0 ? kN / 2 : kN;          // output columns per tile
    const int ntn = NOUT / ncol;
    const int nst = KB / kStage;                        // stages per tile (>= 2)

    extern __shared__ __attribute__((aligned(1024))) uint8_t ring[];
    __shared__ uint32_t aoff[kM];   // activation (or h) row byte offsets
    __shared__ int out_row[kM];     // output rows (-1: none)

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / 4, wn = wave % 4;

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        // ---- decode: tiles of a group are n-tile-major, m-tiles innermost
        const int t = (int)it.t;
        const int eidx = t / ntn;
        const int2 ent = L.entries[eidx];
        const GroupInfo gi = group_info(A, ent.x);
        const int cg = (gi.m + kM - 1) / kM;
        const int bg = eidx - ent.y / kM;
        const int local = t - bg * ntn;
        const int nt = local / cg, mt = local % cg;
        const int m0 = mt * kM;
        const int n0 = nt * ncol;
        const Bank bk = gi.shared ? A.shared : A.routed;

        __syncthreads();   // the previous tile is done with the ring and the row tables
        if (tid < kM) {
            const int r = min(m0 + tid, gi.m - 1);     // rows past the end re-read the last row
            uint32_t o;
            if (PHASE == 0) {
                const int ar = gi.shared ? r : (A.src ? A.src[gi.p0 + r] / A.src_div : gi.p0 + r);
                o = (uint32_t)ar * (uint32_t)(H * 2);
            } else {
                o = (uint32_t)h_row(A, gi, r) * (uint32_t)(I * 2);
            }
            aoff[tid] = o;
            out_row[tid] = m0 + tid < gi.m ? (PHASE == 0 ? h_row(A, gi, m0 + tid)
                                                         : (gi.shared ? m0 + tid : gi.p0 + m0 + tid))
                                           : -1;
        }
        __syncthreads();

        Loads ld;
        {
            const uint8_t* abase = uniform_ptr(PHASE == 0 ? (gi.shared ? A.a_sh : A.a) : A.h);
            const size_t ew = (size_t)gi.e * H * I * 2;   // one expert's matrix, bytes
#pragma unroll
            for (int q = 0; q < kLoads; ++q) {
                const int row0 = 8 * (kLoads * wave + q);   // wave-uniform
                const int row = row0 + lane / 8;
                const uint32_t c16 = (uint32_t)(((lane % 8) ^ swz_key(row)) * 16);
                if (row0 < kM) {
                    ld.base[q] = abase;
                    ld.off[q] = aoff[row] + c16;
                } else {
                    const int j = row - kM;                  // weight row of the tile
                    const void* w = PHASE == 0 ? (row0 - kM < 128 ? bk.wg : bk.wu) : bk.wd;
                    ld.base[q] = uniform_ptr((const uint8_t*)w + ew);
                    ld.off[q] = (uint32_t)(n0 + (PHASE == 0 ? (j & 127) : j)) * (uint32_t)KB + c16;
                }
            }
        }

        f32x16 acc[2] = {f32x16{}, f32x16{}};
        issue_stage(ring, ld, 0, wave);
        issue_stage(ring + kStageBytes, ld, 1, wave);
        // B rows of the wave's blocks: gate/up j = 0 gate rows 32 wn, j = 1 up
        // rows 128 + 32 wn; down rows 64 wn + 32 j
        const int brow0 = kM + (PHASE == 0 ? wn * 32 : wn * 64);
        const int brow1 = kM + (PHASE == 0 ? 128 + wn * 32 : wn * 64 + 32);
        const int arow = wm * 32 + lane % 32;
        for (int s = 0; s < nst; ++s) {
            // stage s landed for every wave (this wave's stage s+1 loads, the
            // newest, may still be in flight); the buffer of stage s-1 is free
            if (s + 1 < nst)
                barrier_vm<kLoads>();
            else
                barrier_vm<0>();
            if (s + 2 < nst) issue_stage(ring + ((s + 2) % kRing) * kStageBytes, ld, s + 2, wave);
            const uint8_t* cur = ring + (s % kRing) * kStageBytes;
            // the next k-step's fragments are read while this one's MFMAs run
            bf16x8 a[2], b0[2], b1[2];
            a[0] = frag16(cur, arow, lane, 0);
            b0[0] = frag16(cur, brow0 + lane % 32, lane, 0);
            b1[0] = frag16(cur, brow1 + lane % 32, lane, 0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c = ks & 1, n = c ^ 1;
                if (ks + 1 < 4) {
                    a[n] = frag16(cur, arow, lane, ks + 1);
                    b0[n] = frag16(cur, brow0 + lane % 32, lane, ks + 1);
                    b1[n] = frag16(cur, brow1 + lane % 32, lane, ks + 1);
                }
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b0[c], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b1[c], acc[1], 0, 0, 0);
            }
        }

        // ---- epilogue: element v of block j is row 32 wm + 8 (v/4) + 4 (lane/32) + v%4,
        // column lane%32 of the block
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = wm * 32 + 8 * (v / 4) + 4 * (lane / 32) + v % 4;
            const int orow = out_row[r];
            if (orow < 0) continue;
            if (PHASE == 0) {
                ((uint16_t*)A.h)[(size_t)orow * I + n0 + wn * 32 + lane % 32] =
                    (uint16_t)f32_to_bf16_bits(silu_mul(acc[0][v], acc[1][v]));
            } else {
                void* yb = gi.shared ? A.y_sh : A.y;
                const int ybf = gi.shared ? A.y_sh_bf16 : A.y_bf16;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const size_t o = (size_t)orow * H + n0 + wn * 64 + 32 * j + lane % 32;
                    if (ybf) ((uint16_t*)yb)[o] = (uint16_t)f32_to_bf16_bits(acc[j][v]);
                    else ((float*)yb)[o] = acc[j][v];
                }
            }
        }
    }
}

constexpr size_t kMidLds = (size_t)kRing * kStageBytes;

template <int PHASE>
static hipError_t launch_mid_t(const GArgs& A, const TileList& L, hipStream_t s) {
    static DeviceCache cache;
    const int grid = per_device(cache, [] {
        (void)hipFuncSetAttribute((const void*)mid_kernel<PHASE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)kMidLds);
        return device_cu_count();   // one 512-thread workgroup per CU (LDS-limited)
    });
    hipLaunchKernelGGL(mid_kernel<PHASE>, dim3(grid), dim3(512), kMidLds, s, A, L);
    return hipGetLastError();
}

hipError_t launch_mid_gateup(const GArgs& A, const TileList& L, hipStream_t s) { return launch_mid_t<0>(A, L, s); }
hipError_t launch_mid_down(const GArgs& A, const TileList& L, hipStream_t s) { return launch_mid_t<1>(A, L, s); }

}  // namespace moe
