// Grouped expert FFN with MXFP4 weights, large tiles for groups with many
// rows ("DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1: at prefill
// sizes each routed expert sees hundreds to thousands of rows and the GEMMs
// are compute-bound; the FP4 weights of the pages' Blackwell deployment, "How
// DeepSeek inference works", deployment lever table).
//
// Tile: 256 rows x 256 MFMA columns (gate/up: 128 gate + 128 up weight rows
// of the same 128 h columns; down: 256 output columns), 8 waves (2 along M x
// 4 along N), each 128 rows x 64 columns, K staged 128 values at a time.
// The MFMA is v_mfma_scale_f32_16x16x128_f8f6f4 in transposed form: the row
// operand is a block of 16 weight rows in FP4, the column operand 16 tokens
// in FP8, and each carries its E8M0 exponent per lane and 32-K block, so
// partial products join the accumulator inside the MFMA with no per-block
// rescaling on the vector ALU (the e4m3 kernel's fp32 block scales need one
// FMA per accumulator and block).  Operand layouts (measured on the device):
// FP4 lane group g holds K 32g..32g+31 of its row (16 bytes), FP8 lane group
// g holds K 16g..16g+15 and 64+16g..64+16g+15 (two 16-byte pieces);
// exponents are those of K block g.
//
// A stage is 48 KiB (256 token rows x 128 bytes, 256 weight rows x 64 bytes)
// plus each row's exponent dword (the four 32-K blocks of the stage), moved
// by direct global->LDS loads.  Three stages rotate through LDS, so two are
// in flight while one is consumed; waves wait on their own loads with an
// explicit vmcnt and meet at a plain barrier (a full fence would also wait
// for the stage that should stay in flight).  LDS rows are XOR-swizzled in
// 16-byte chunks so that the 16 lanes of a fragment read hit all banks once:
// key (r & 7) ^ ((r >> 3) & 1) for 128-byte token rows, (r >> 2) & 3 for
// 64-byte weight rows.
//
// Epilogues: gate/up applies SwiGLU and writes h as MXFP8 (a wave holds 32 h
// columns of a row, exactly one 32-column block); down writes y in fp32 or
// bf16.  Tiles of a group are ordered n-tile-major with its m-tiles
// innermost (as in gffn_big.hip), so the m-tiles that share a weight tile
// run side by side on one die.
#include "gffn_common.h"

namespace moe {

namespace {

constexpr int kXM = 256, kXN = 256;                     // tile rows, MFMA columns
constexpr int kXAB = kXM * 128;                          // token bytes per stage (fp8, 128 K)
constexpr int kXBB = kXN * 64;                           // weight bytes per stage (fp4, 128 K)
constexpr int kXStage = kXAB + kXBB;                     // 48 KiB
constexpr int kXRing = 3;                                // stages in LDS
constexpr int kXDma = 4 + 2 + 1;                         // direct loads per wave and stage

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int key8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int key4(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ const uint8_t* wave_ptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

struct XSmem {
    uint8_t* stage;       // [3][48 KiB]
    uint32_t* ea;         // [3][256] token exponent dwords of a stage
    uint32_t* eb;         // [3][256] weight exponent dwords of a stage
    uint32_t* aoff;       // [256] token row byte offsets (from the activation / h base)
    uint32_t* aeoff;      // [256] token row exponent byte offsets
    int* out_row;         // [256] output rows (-1: none)
};

constexpr size_t kXLds = (size_t)kXRing * kXStage + 2 * kXRing * kXM * 4 + 3 * kXM * 4 + kXM * 4;

}  // namespace

// PHASE 0: gate/up (+SwiGLU, MXFP8 h); PHASE 1: down.
template <int PHASE>
__global__ __launch_bounds__(512) void mxbig_kernel(GArgs A, TileList L) {
    const int H = A.H, I = A.I;
    const int K = PHASE == 0 ? H : I;                  // reduction length
    const int NOUT = PHASE == 0 ? I : H;                // output columns of the phase
    const int ncol = PHASE == 0 ? kXN / 2 : kXN;        // output columns per tile
    const int ntn = NOUT / ncol;
    const int nstages = K / 128;

    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    XSmem S;
    S.stage = smem;
    S.ea = (uint32_t*)(smem + (size_t)kXRing * kXStage);
    S.eb = S.ea + kXRing * kXM;
    S.aoff = S.eb + kXRing * kXM;
    S.aeoff = S.aoff + kXM;
    S.out_row = (int*)(S.aeoff + kXM);

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / 4, wn = wave % 4;
    const int g = lane / 16;                        // K block of the lane within an MFMA
    const uint32_t esh = 8u * g;

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        // ---- decode: tiles of a group are n-tile-major, m-tiles innermost
        const int t = (int)it.t;
        const int eidx = t / ntn;
        const int2 ent = L.entries[eidx];
        const GroupInfo gi = group_info(A, ent.x);
        const int cg = (gi.m + kXM - 1) / kXM;
        const int bg = eidx - ent.y / kXM;
        const int local = t - bg * ntn;
        const int nt = local / cg, mt = local % cg;
        const int m0 = mt * kXM;
        const int n0 = nt * ncol;
        const Bank bk = gi.shared ? A.shared : A.routed;

        wait_vm<0>();      // the previous tile's stores: the stage accounting below counts loads only
        __syncthreads();   // the previous tile is done with LDS
        if (tid < kXM) {
            const int r = min(m0 + tid, gi.m - 1);      // rows past the end re-read the last row
            uint32_t ar;
            if (PHASE == 0) {
                ar = gi.shared ? (uint32_t)r : (uint32_t)(A.src ? A.src[gi.p0 + r] / A.src_div : gi.p0 + r);
            } else {
                ar = (uint32_t)h_row(A, gi, r);
            }
            S.aoff[tid] = ar * (uint32_t)K;
            S.aeoff[tid] = ar * (uint32_t)(K / 32);
            S.out_row[tid] = (m0 + tid < gi.m) ? (PHASE == 0 ? h_row(A, gi, m0 + tid)
                                                             : (gi.shared ? m0 + tid : gi.p0 + m0 + tid))
                                               : -1;
        }
        __syncthreads();

        // ---- this lane's direct loads: 4 token chunks, 2 weight chunks, 1 exponent dword
        const uint8_t* abase = wave_ptr(PHASE == 0 ? (gi.shared ? A.a_sh : A.a) : A.h);
        const uint8_t* aebase = wave_ptr(PHASE == 0 ? (const void*)(gi.shared ? A.a_sh_scale : A.a_scale)
                                                    : (const void*)A.h_scale);
        uint32_t ao[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 8 * (4 * wave + q) + lane / 8;
            ao[q] = S.aoff[row] + (uint32_t)((((lane % 8) ^ key8(row))) << 4);
        }
        // weight rows of the tile: gate/up rows 0..127 gate, 128..255 up (waves 4-7); down: all of W_down
        const int brow0 = 16 * (2 * wave);
        const int wsel = PHASE == 0 ? (wave >= 4) : 0;
        const uint8_t* wbase = wave_ptr((const uint8_t*)(PHASE == 0 ? (wsel ? bk.wu : bk.wg) : bk.wd) +
                                        (size_t)gi.e * H * I / 2);
        uint32_t bo[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = brow0 + 16 * q + lane / 4;               // 0 .. 255
            const int wrow = n0 + (PHASE == 0 ? (row & 127) : row);
            bo[q] = (uint32_t)wrow * (uint32_t)(K / 2) + (uint32_t)((((lane % 4) ^ key4(row))) << 4);
        }
        // exponent dwords: waves 0-3 token rows 64 w + l, waves 4-7 weight rows 64 (w - 4) + l
        const uint8_t* ebase;
        uint32_t eo;
        if (wave < 4) {
            ebase = aebase;
            eo = S.aeoff[64 * wave + lane];
        } else {
            const int row = 64 * (wave - 4) + lane;
            const int wrow = n0 + (PHASE == 0 ? (row & 127) : row);
            const void* eb = PHASE == 0 ? (row < 128 ? (const void*)bk.sg : (const void*)bk.su) : (const void*)bk.sd;
            ebase = wave_ptr((const uint8_t*)eb + (size_t)gi.e * H * I / 32);
            eo = (uint32_t)wrow * (uint32_t)(K / 32);
        }
        // gate/up waves 4-5 hold gate exponent rows 0..127, 6-7 up rows: per-wave bases are uniform
        auto issue = [&](int s) {
            uint8_t* st = S.stage + (s % kXRing) * kXStage;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_global_load_lds((const void*)(abase + ao[q] + s * 128),
                                                 (lds_void*)(st + (4 * wave + q) * 1024), 16, 0, 0);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                __builtin_amdgcn_global_load_lds((const void*)(wbase + bo[q] + s * 64),
                                                 (lds_void*)(st + kXAB + (2 * wave + q) * 1024), 16, 0, 0);
            uint32_t* ed = (wave < 4 ? S.ea + 64 * wave : S.eb + 64 * (wave - 4)) + (s % kXRing) * kXM;
            __builtin_amdgcn_global_load_lds((const void*)(ebase + eo + s * 4), (lds_void*)ed, 4, 0, 0);
        };

        f32x4 acc[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        issue(0);
        if (nstages > 1) issue(1);
        for (int s = 0; s < nstages; ++s) {
            // this wave's loads of stage s done (stage s+1's may stay in flight), then everyone's
            if (s + 1 < nstages) wait_vm<kXDma>();
            else wait_vm<0>();
            // compiler-only fences around the bare barrier (no waitcnt is
            // emitted): LDS reads of stage s stay below it, writes of stage
            // s-1 above it
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            // the buffer of stage s-1, which every wave has finished, takes stage s+2
            if (s + 2 < nstages) issue(s + 2);

            const int b = s % kXRing;
            const uint8_t* As = S.stage + b * kXStage;
            const uint8_t* Bs = As + kXAB;
            const uint32_t* ea = S.ea + b * kXM;
            const uint32_t* eb = S.eb + b * kXM;
            // weight blocks j: gate/up j<2 gate rows wn*32+16j, j>=2 up rows 128+wn*32+16(j-2); down wn*64+16j
            i32x8 wf[4];
            uint32_t ew[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = (PHASE == 0 ? (j < 2 ? wn * 32 + 16 * j : 128 + wn * 32 + 16 * (j - 2)) : wn * 64 + 16 * j) +
                              lane % 16;
                const i32x4 v = *(const i32x4*)(Bs + r * 64 + ((g ^ key4(r)) << 4));
                wf[j] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
                ew[j] = eb[r] >> esh;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wm * 128 + 16 * i + lane % 16;
                const uint8_t* row = As + r * 128;
                const i32x4 lo = *(const i32x4*)(row + ((g ^ key8(r)) << 4));
                const i32x4 hi = *(const i32x4*)(row + (((4 + g) ^ key8(r)) << 4));
                const i32x8 x = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const uint32_t et = ea[r] >> esh;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], x, acc[i][j], 4, 0, 0, (int)ew[j],
                                                                                0, (int)et);
            }
        }

        // ---- epilogue.  Element (i, j, q) of the wave's accumulator: token
        // wm*128 + 16 i + lane%16, MFMA column (weight row of block j) 4 g + q.
        if (PHASE == 0) {
            uint8_t* he = (uint8_t*)A.h_scale;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float hv[2][4];
                float mx = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        hv[j][q] = silu_mul(acc[i][j][q], acc[i][j + 2][q]);
                        mx = fmaxf(mx, fabsf(hv[j][q]));
                    }
                // the row's 32 h columns of this wave sit in the four lanes of lane%16
                mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                const uint32_t E = mx_e8m0_for_e4m3(mx);
                const float f = mx_inv_scale(E);
                const int hr = S.out_row[wm * 128 + 16 * i + lane % 16];
                if (hr < 0) continue;
                const int c0 = n0 + wn * 32;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    *(uint32_t*)(A.h + (size_t)hr * I + c0 + 16 * j + 4 * g) =
                        f32x4_to_e4m3x4(hv[j][0] * f, hv[j][1] * f, hv[j][2] * f, hv[j][3] * f);
                if (g == 0) he[(size_t)hr * (I / 32) + c0 / 32] = (uint8_t)E;
            }
        } else {
            void* yb = gi.shared ? A.y_sh : A.y;
            const int ybf = gi.shared ? A.y_sh_bf16 : A.y_bf16;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int yr = S.out_row[wm * 128 + 16 * i + lane % 16];
                if (yr < 0) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const size_t o = (size_t)yr * H + n0 + wn * 64 + 16 * j + 4 * g;
                    const f32x4 v = acc[i][j];
                    if (ybf) {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *(uint2*)((uint16_t*)yb + o) = make_uint2(lo, hi);
                    } else {
                        *(f32x4*)((float*)yb + o) = v;
                    }
                }
            }
        }
    }
}

template <int PHASE>
static hipError_t launch_mxbig_t(const GArgs& A, const TileList& L, hipStream_t s) {
    static DeviceCache cache;
    const int grid = per_device(cache, [] {
        hipFuncSetAttribute((const void*)mxbig_kernel<PHASE>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kXLds);
        return device_cu_count();   // one 512-thread workgroup per CU (LDS-limited)
    });
    hipLaunchKernelGGL((mxbig_kernel<PHASE>), dim3(grid), dim3(512), kXLds, s, A, L);
    return hipGetLastError();
}

hipError_t launch_mxbig_gateup(const GArgs& A, const TileList& L, hipStream_t s) { return launch_mxbig_t<0>(A, L, s); }
hipError_t launch_mxbig_down(const GArgs& A, const TileList& L, hipStream_t s) { return launch_mxbig_t<1>(A, L, s); }

}  // namespace moe
