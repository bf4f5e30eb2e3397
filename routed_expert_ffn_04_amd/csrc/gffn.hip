// Grouped expert FFN on gfx950 matrix cores ("DeepSeek V3/R1 Inference
// Efficiency (2)", section 2.3.1: routed expert GEMM "up & gate"
// [7168, 4096] and "down" [2048, 7168] per group, shared expert GEMMs, and
// the SwiGLU operator between them; section 2.4.1 for the small-m decode
// shapes).
//
// Phase 1 (gate/up): for a tile of BM rows of one group and BN columns of I,
//   G = A Wg, U = A Wu over K = H on MFMA, then h = silu(G) * U in the
//   epilogue, rounded to bf16 or quantised to e4m3 per 1x128 (the SwiGLU
//   operator is fused into the producing GEMM instead of being a separate
//   memory-bound pass).  A rows are gathered through src / src_div, so no
//   permuted copy of the tokens is ever written.
// Phase 2 (down): y = h Wd over K = I.
//
// Scheduling: a single-workgroup kernel reads the device-resident offsets
// and writes the list of (group, first row) m-tiles; the GEMM grids are
// (n-tiles, upper bound of m-tiles) and surplus workgroups exit at once, so
// the per-expert counts never travel to the host.
//
// Operands are K-contiguous in both A and the output-major weights, which is
// the layout every MFMA operand wants (lane = row or column, a run of
// consecutive k per lane): 16-byte global loads, no transposes.
//   bf16 : v_mfma_f32_16x16x32_bf16   (k = 32 per instruction)
//   e4m3 : v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (k = 128 =
//          one scaling block); the fp32 block scales are applied to each
//          block's partial product before it joins the fp32 accumulator.
//   f32  : v_mfma_f32_16x16x4_f32
#include "common.h"
#include "internal.h"

namespace moe {

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

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

struct GArgs {
    const uint8_t* a; const float* a_scale; const int32_t* src; int src_div;
    const uint8_t* a_sh; const float* a_sh_scale;
    const int32_t* offsets; int G; int R_max; int S;
    Bank routed, shared;
    int H, I;
    uint8_t* h; float* h_scale;        // [R_max + S][I], [R_max + S][I/128]
    void* y; void* y_sh; int y_bf16;
    const int2* tiles; const int* ntiles;
};

constexpr int kBM = 64;      // rows per tile
constexpr int kBN = 128;     // output columns per tile
constexpr int kBKB = 128;    // K bytes staged per step
constexpr int kPad = 16;     // LDS row padding (bytes)
constexpr int kRowB = kBKB + kPad;

// ---------------------------------------------------------------- tile list
// Rows per group are clamped to [0, R_max - offsets[g]] and the list to
// maxt entries, so malformed offsets cannot send a tile out of bounds.
__global__ __launch_bounds__(1024) void gffn_build_tiles(const int32_t* __restrict__ offsets, int G, int S,
                                                         int R_max, int BM, int maxt, int2* __restrict__ tiles,
                                                         int* __restrict__ ntiles) {
    __shared__ int wsum[16];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    if (tid == 0) carry = 0;
    __syncthreads();
    const int ngroups = G + (S > 0 ? 1 : 0);
    for (int g0 = 0; g0 < ngroups; g0 += 1024) {
        const int g = g0 + tid;
        int m = 0;
        if (g < G) {
            const int p0 = min(max(offsets[g], 0), R_max);
            m = min(max(offsets[g + 1] - p0, 0), R_max - p0);
        } else if (g == G && S > 0) {
            m = S;
        }
        const int nt = (m + BM - 1) / BM;
        int v = nt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(v, d, kWave);
            if (lane >= d) v += o;
        }
        if (lane == kWave - 1) wsum[w] = v;
        __syncthreads();
        int base = carry;
        for (int i = 0; i < w; ++i) base += wsum[i];
        base += v - nt;
        for (int i = 0; i < nt && base + i < maxt; ++i) tiles[base + i] = make_int2(g, i * BM);
        __syncthreads();
        if (tid == 1023) carry = base + nt;
        __syncthreads();
    }
    if (tid == 0) *ntiles = min(carry, maxt);
}

// ---------------------------------------------------------------- helpers
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

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

// Copy a [rows][kBKB] byte tile from global (row pointers) into LDS.
// 16-byte chunks; rows with a null pointer are zero-filled.
template <int ROWS>
__device__ __forceinline__ void stage_rows(uint8_t* lds, const uint8_t* const* rowp, size_t koff, int tid) {
    constexpr int CHUNKS = ROWS * (kBKB / 16);
#pragma unroll
    for (int i = tid; i < CHUNKS; i += 256) {
        const int r = i / (kBKB / 16), c = i % (kBKB / 16);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (rowp[r]) v = *(const uint4*)(rowp[r] + koff + c * 16);
        *(uint4*)(lds + r * kRowB + c * 16) = v;
    }
}

// ---------------------------------------------------------------- phase 1
template <int DT>
__global__ __launch_bounds__(256) void gffn_gateup_kernel(GArgs A) {
    using O = Op<DT>;
    if ((int)blockIdx.y >= *A.ntiles) return;
    const int2 tl = A.tiles[blockIdx.y];
    const GroupInfo gi = group_info(A, tl.x);
    const int m0 = tl.y;
    const int n0 = blockIdx.x * kBN;
    const int H = A.H, I = A.I, nkb = H / 128;
    const Bank& bk = gi.shared ? A.shared : A.routed;

    __shared__ __attribute__((aligned(16))) uint8_t As[kBM * kRowB];
    __shared__ __attribute__((aligned(16))) uint8_t Bg[kBN * kRowB];
    __shared__ __attribute__((aligned(16))) uint8_t Bu[kBN * kRowB];
    __shared__ const uint8_t* arow[kBM];
    __shared__ const uint8_t* grow[kBN];
    __shared__ const uint8_t* urow[kBN];
    __shared__ int hrow[kBM];
    __shared__ float sA[kBM];
    __shared__ const float* sArow[kBM];
    __shared__ float amax_red[2][kBM];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    if (tid < kBM) {
        const int r = m0 + tid;
        const uint8_t* p = nullptr;
        const float* ps = nullptr;
        int hr = -1;
        if (r < gi.m) {
            if (gi.shared) {
                p = A.a_sh + (size_t)r * H * O::EB;
                if (DT == DT_E4M3) ps = A.a_sh_scale + (size_t)r * nkb;
                hr = A.R_max + r;
            } else {
                const int pp = gi.p0 + r;
                const int ar = A.src ? A.src[pp] / A.src_div : pp;
                p = A.a + (size_t)ar * H * O::EB;
                if (DT == DT_E4M3) ps = A.a_scale + (size_t)ar * nkb;
                hr = pp;
            }
        }
        arow[tid] = p;
        sArow[tid] = ps;
        hrow[tid] = hr;
    }
    if (tid < kBN) {
        const size_t wrow = (size_t)gi.e * I + n0 + tid;
        grow[tid] = (const uint8_t*)bk.wg + wrow * H * O::EB;
        urow[tid] = (const uint8_t*)bk.wu + wrow * H * O::EB;
    }
    __syncthreads();

    constexpr int MB = 2, NB = 4;     // 16x16 blocks per wave: 32 rows x 64 cols
    f32x4 accg[MB][NB], accu[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) accg[i][j] = accu[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KB = H * O::EB;         // bytes of K per row
    for (int k0 = 0; k0 < KB; k0 += kBKB) {
        stage_rows<kBM>(As, arow, k0, tid);
        stage_rows<kBN>(Bg, grow, k0, tid);
        stage_rows<kBN>(Bu, urow, k0, tid);
        float sgv = 1.f, suv = 1.f;
        if (DT == DT_E4M3) {
            if (tid < kBM) sA[tid] = sArow[tid] ? sArow[tid][k0 / 128] : 0.f;
            const size_t sidx = ((size_t)gi.e * (I / 128) + n0 / 128) * nkb + k0 / 128;
            sgv = bk.sg[sidx];
            suv = bk.su[sidx];
        }
        __syncthreads();
        constexpr int KSTEPS = kBKB / (O::KI * O::EB);
        if (DT == DT_E4M3) {
            const uint8_t* ap[MB];
            float sa[MB][4];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int rb = wm * 32 + i * 16;
                ap[i] = As + (rb + lane % 16) * kRowB + (lane / 16) * O::LB;
#pragma unroll
                for (int q = 0; q < 4; ++q) sa[i][q] = sA[rb + 4 * (lane / 16) + q];
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int cb = wn * 64 + j * 16;
                const uint8_t* gp = Bg + (cb + lane % 16) * kRowB + (lane / 16) * O::LB;
                const uint8_t* up = Bu + (cb + lane % 16) * kRowB + (lane / 16) * O::LB;
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 tg = O::mma(ap[i], gp, z);
                    const f32x4 tu = O::mma(ap[i], up, z);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        accg[i][j][q] = __builtin_fmaf(tg[q], sa[i][q] * sgv, accg[i][j][q]);
                        accu[i][j][q] = __builtin_fmaf(tu[q], sa[i][q] * suv, accu[i][j][q]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const int kb = ks * O::KI * O::EB + (lane / 16) * O::LB;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int cb = wn * 64 + j * 16;
                    const uint8_t* gp = Bg + (cb + lane % 16) * kRowB + kb;
                    const uint8_t* up = Bu + (cb + lane % 16) * kRowB + kb;
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        const uint8_t* ap = As + (wm * 32 + i * 16 + lane % 16) * kRowB + kb;
                        accg[i][j] = O::mma(ap, gp, accg[i][j]);
                        accu[i][j] = O::mma(ap, up, accu[i][j]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // epilogue: h = silu(g) * u, then round / quantise and store
    float hv[MB][NB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[i][j][q] = silu_mul(accg[i][j][q], accu[i][j][q]);

    if (DT == DT_E4M3) {
        // amax over the 128 columns of the tile for every row
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float mx = 0.f;
#pragma unroll
                for (int j = 0; j < NB; ++j) mx = fmaxf(mx, fabsf(hv[i][j][q]));
#pragma unroll
                for (int s = 8; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s, kWave));
                if (lane % 16 == 0) amax_red[wn][wm * 32 + i * 16 + 4 * (lane / 16) + q] = mx;
            }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = wm * 32 + i * 16 + 4 * (lane / 16) + q;
            const int hr = hrow[r];
            if (hr < 0) continue;
            float s = 1.f;
            if (DT == DT_E4M3) {
                const float amax = fmaxf(amax_red[0][r], amax_red[1][r]);
                s = amax > 0.f ? amax / 448.0f : 1.0f;
                if (wn == 0 && lane % 16 == 0) A.h_scale[(size_t)hr * (I / 128) + n0 / 128] = s;
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int c = n0 + wn * 64 + j * 16 + lane % 16;
                const float v = hv[i][j][q];
                if (DT == DT_F32) ((float*)A.h)[(size_t)hr * I + c] = v;
                else if (DT == DT_BF16) ((uint16_t*)A.h)[(size_t)hr * I + c] = (uint16_t)f32_to_bf16_bits(v);
                else A.h[(size_t)hr * I + c] = (uint8_t)f32_to_e4m3(v / s);
            }
        }
}

// ---------------------------------------------------------------- phase 2
template <int DT>
__global__ __launch_bounds__(256) void gffn_down_kernel(GArgs A) {
    using O = Op<DT>;
    if ((int)blockIdx.y >= *A.ntiles) return;
    const int2 tl = A.tiles[blockIdx.y];
    const GroupInfo gi = group_info(A, tl.x);
    const int m0 = tl.y;
    const int n0 = blockIdx.x * kBN;
    const int H = A.H, I = A.I, nkb = I / 128;
    const Bank& bk = gi.shared ? A.shared : A.routed;

    __shared__ __attribute__((aligned(16))) uint8_t As[kBM * kRowB];
    __shared__ __attribute__((aligned(16))) uint8_t Bd[kBN * kRowB];
    __shared__ const uint8_t* arow[kBM];
    __shared__ const uint8_t* drow[kBN];
    __shared__ int yrow[kBM];
    __shared__ float sA[kBM];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    if (tid < kBM) {
        const int r = m0 + tid;
        const uint8_t* p = nullptr;
        int yr = -1;
        if (r < gi.m) {
            const int hr = gi.shared ? A.R_max + r : gi.p0 + r;
            p = A.h + (size_t)hr * I * O::EB;
            yr = gi.shared ? r : gi.p0 + r;
        }
        arow[tid] = p;
        yrow[tid] = yr;
    }
    if (tid < kBN) drow[tid] = (const uint8_t*)bk.wd + ((size_t)gi.e * H + n0 + tid) * I * O::EB;
    __syncthreads();

    constexpr int MB = 2, NB = 4;
    f32x4 acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KB = I * O::EB;
    for (int k0 = 0; k0 < KB; k0 += kBKB) {
        stage_rows<kBM>(As, arow, k0, tid);
        stage_rows<kBN>(Bd, drow, k0, tid);
        float sdv = 1.f;
        if (DT == DT_E4M3) {
            if (tid < kBM) {
                const int r = m0 + tid;
                float v = 0.f;
                if (r < gi.m) {
                    const int hr = gi.shared ? A.R_max + r : gi.p0 + r;
                    v = A.h_scale[(size_t)hr * nkb + k0 / 128];
                }
                sA[tid] = v;
            }
            sdv = bk.sd[((size_t)gi.e * (H / 128) + n0 / 128) * nkb + k0 / 128];
        }
        __syncthreads();
        constexpr int KSTEPS = kBKB / (O::KI * O::EB);
        if (DT == DT_E4M3) {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int rb = wm * 32 + i * 16;
                const uint8_t* ap = As + (rb + lane % 16) * kRowB + (lane / 16) * O::LB;
                float sc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) sc[q] = sA[rb + 4 * (lane / 16) + q] * sdv;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint8_t* bp = Bd + (wn * 64 + j * 16 + lane % 16) * kRowB + (lane / 16) * O::LB;
                    const f32x4 t = O::mma(ap, bp, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(t[q], sc[q], acc[i][j][q]);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const int kb = ks * O::KI * O::EB + (lane / 16) * O::LB;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const uint8_t* bp = Bd + (wn * 64 + j * 16 + lane % 16) * kRowB + kb;
#pragma unroll
                    for (int i = 0; i < MB; ++i) {
                        const uint8_t* ap = As + (wm * 32 + i * 16 + lane % 16) * kRowB + kb;
                        acc[i][j] = O::mma(ap, bp, acc[i][j]);
                    }
                }
            }
        }
        __syncthreads();
    }

    void* yb = gi.shared ? A.y_sh : A.y;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = wm * 32 + i * 16 + 4 * (lane / 16) + q;
            const int yr = yrow[r];
            if (yr < 0) continue;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int c = n0 + wn * 64 + j * 16 + lane % 16;
                if (A.y_bf16) ((uint16_t*)yb)[(size_t)yr * H + c] = (uint16_t)f32_to_bf16_bits(acc[i][j][q]);
                else ((float*)yb)[(size_t)yr * H + c] = acc[i][j][q];
            }
        }
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int max_mtiles(int R_max, int G, int S) {
    return (R_max + kBM - 1) / kBM + G + (S + kBM - 1) / kBM;
}

size_t gffn_ws_bytes(int R_max, int G, int S, int H, int I, int dt) {
    const size_t rows = (size_t)R_max + S;
    const int eb = dt == DT_F32 ? 4 : dt == DT_BF16 ? 2 : 1;
    size_t b = align256(rows * I * eb);
    b += align256(rows * (I / 128) * sizeof(float));
    b += align256((size_t)max_mtiles(R_max, G, S) * sizeof(int2));
    b += align256(sizeof(int));
    return b;
}

hipError_t launch_gffn(const GffnProblem& p, void* ws, hipStream_t s) {
    GArgs A;
    A.a = (const uint8_t*)p.a; A.a_scale = p.a_scale; A.src = p.src; A.src_div = p.src_div;
    A.a_sh = (const uint8_t*)p.a_sh; A.a_sh_scale = p.a_sh_scale;
    A.offsets = p.offsets; A.G = p.G; A.R_max = p.R_max; A.S = p.has_shared ? p.S : 0;
    A.routed = p.routed; A.shared = p.shared; A.H = p.H; A.I = p.I;
    A.y = p.y; A.y_sh = p.y_sh; A.y_bf16 = p.y_bf16;
    const size_t rows = (size_t)p.R_max + A.S;
    const int eb = p.dt == DT_F32 ? 4 : p.dt == DT_BF16 ? 2 : 1;
    uint8_t* w = (uint8_t*)ws;
    A.h = w; w += align256(rows * p.I * eb);
    A.h_scale = (float*)w; w += align256(rows * (p.I / 128) * sizeof(float));
    int2* tiles = (int2*)w; w += align256((size_t)max_mtiles(p.R_max, p.G, A.S) * sizeof(int2));
    int* ntiles = (int*)w;
    A.tiles = tiles; A.ntiles = ntiles;
    const int mt = max_mtiles(p.R_max, p.G, A.S);

    hipLaunchKernelGGL(gffn_build_tiles, dim3(1), dim3(1024), 0, s, p.offsets, p.G, A.S, p.R_max, kBM, mt, tiles,
                       ntiles);
    dim3 g1(p.I / kBN, mt), g2(p.H / kBN, mt);
    switch (p.dt) {
        case DT_F32:
            hipLaunchKernelGGL(gffn_gateup_kernel<DT_F32>, g1, dim3(256), 0, s, A);
            hipLaunchKernelGGL(gffn_down_kernel<DT_F32>, g2, dim3(256), 0, s, A);
            break;
        case DT_BF16:
            hipLaunchKernelGGL(gffn_gateup_kernel<DT_BF16>, g1, dim3(256), 0, s, A);
            hipLaunchKernelGGL(gffn_down_kernel<DT_BF16>, g2, dim3(256), 0, s, A);
            break;
        default:
            hipLaunchKernelGGL(gffn_gateup_kernel<DT_E4M3>, g1, dim3(256), 0, s, A);
            hipLaunchKernelGGL(gffn_down_kernel<DT_E4M3>, g2, dim3(256), 0, s, A);
            break;
    }
    return hipGetLastError();
}

}  // namespace moe
