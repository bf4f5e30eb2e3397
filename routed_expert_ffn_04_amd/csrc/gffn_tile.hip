// Grouped expert FFN, LDS-tiled MFMA kernels (any operand type): tiles of
// 64 rows x 128 output columns, K staged through LDS 128 bytes at a time.
// "DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1: the routed and
// shared expert "up & gate" [H, 2I] and "down" [I, H] GEMMs, with the SwiGLU
// operator fused into the gate/up epilogue.
//
// Persistent workgroups claim (m-tile, n-tile) pairs from a device-built list
// (gffn.hip), so per-expert row counts never leave the GPU.
//
// MFMA operands are K-contiguous on both sides (activation rows and the
// output-major weights): lane = row/column, consecutive k per lane.
//   bf16 : v_mfma_f32_16x16x32_bf16
//   e4m3 : v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales; one
//          instruction covers one 128-wide scaling block, and its partial
//          product is multiplied by (activation scale x weight scale) before
//          it joins the fp32 accumulator
//   f32  : v_mfma_f32_16x16x4_f32
#include "gffn_common.h"

namespace moe {

constexpr int kBM = 64;      // rows per tile
constexpr int kBN = 128;     // output columns per tile
constexpr int kBKB = 128;    // K bytes staged per step
constexpr int kPad = 16;     // LDS row padding (bytes)
constexpr int kRowB = kBKB + kPad;

// Copy a [ROWS][kBKB] byte tile from global (row pointers) into LDS.
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
__global__ __launch_bounds__(256) void tile_gateup_kernel(GArgs A, TileList L) {
    using O = Op<DT>;
    const int H = A.H, I = A.I, nkb = H / 128;
    const int ntn = I / kBN;

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

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        const int t = (int)it.t;
        __syncthreads();   // the previous tile's epilogue is done with the LDS tables
        const int2 tl = L.entries[t / ntn];
        const GroupInfo gi = group_info(A, tl.x);
        const int m0 = tl.y;
        const int n0 = (t % ntn) * kBN;
        const Bank& bk = gi.shared ? A.shared : A.routed;

        if (tid < kBM) {
            const int r = m0 + tid;
            const uint8_t* p = nullptr;
            const float* ps = nullptr;
            int hr = -1;
            if (r < gi.m) {
                if (gi.shared) {
                    p = A.a_sh + (size_t)r * H * O::EB;
                    if (DT == DT_E4M3) ps = A.a_sh_scale + (size_t)r * nkb;
                } else {
                    const int pp = gi.p0 + r;
                    const int ar = A.src ? A.src[pp] / A.src_div : pp;
                    p = A.a + (size_t)ar * H * O::EB;
                    if (DT == DT_E4M3) ps = A.a_scale + (size_t)ar * nkb;
                }
                hr = h_row(A, gi, r);
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
}

// ---------------------------------------------------------------- phase 2
template <int DT>
__global__ __launch_bounds__(256) void tile_down_kernel(GArgs A, TileList L) {
    using O = Op<DT>;
    const int H = A.H, I = A.I, nkb = I / 128;
    const int ntn = H / kBN;

    __shared__ __attribute__((aligned(16))) uint8_t As[kBM * kRowB];
    __shared__ __attribute__((aligned(16))) uint8_t Bd[kBN * kRowB];
    __shared__ const uint8_t* arow[kBM];
    __shared__ const uint8_t* drow[kBN];
    __shared__ int yrow[kBM];
    __shared__ int hrs[kBM];
    __shared__ float sA[kBM];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        const int t = (int)it.t;
        __syncthreads();   // the previous tile's epilogue is done with the LDS tables
        const int2 tl = L.entries[t / ntn];
        const GroupInfo gi = group_info(A, tl.x);
        const int m0 = tl.y;
        const int n0 = (t % ntn) * kBN;
        const Bank& bk = gi.shared ? A.shared : A.routed;

        if (tid < kBM) {
            const int r = m0 + tid;
            const uint8_t* p = nullptr;
            int yr = -1, hr = -1;
            if (r < gi.m) {
                hr = h_row(A, gi, r);
                p = A.h + (size_t)hr * I * O::EB;
                yr = gi.shared ? r : gi.p0 + r;
            }
            arow[tid] = p;
            yrow[tid] = yr;
            hrs[tid] = hr;
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
                if (tid < kBM) sA[tid] = hrs[tid] >= 0 ? A.h_scale[(size_t)hrs[tid] * nkb + k0 / 128] : 0.f;
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
                        const f32x4 tq = O::mma(ap, bp, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(tq[q], sc[q], acc[i][j][q]);
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
                    if (gi.shared ? A.y_sh_bf16 : A.y_bf16) ((uint16_t*)yb)[(size_t)yr * H + c] = (uint16_t)f32_to_bf16_bits(acc[i][j][q]);
                    else ((float*)yb)[(size_t)yr * H + c] = acc[i][j][q];
                }
            }
    }
}

// ---------------------------------------------------------------- launchers
template <class K>
static int persistent_grid(K kernel, int lds_dynamic) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds_dynamic) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return per_cu * device_cu_count();
}

hipError_t launch_tile_gateup(int dt, const GArgs& A, const TileList& L, int bm, hipStream_t s) {
    (void)bm;
    switch (dt) {
        case DT_F32: {
            static DeviceCache c_;
            const int g = per_device(c_, [] { return persistent_grid(tile_gateup_kernel<DT_F32>, 0); });
            hipLaunchKernelGGL(tile_gateup_kernel<DT_F32>, dim3(g), dim3(256), 0, s, A, L);
            break;
        }
        case DT_BF16: {
            static DeviceCache c_;
            const int g = per_device(c_, [] { return persistent_grid(tile_gateup_kernel<DT_BF16>, 0); });
            hipLaunchKernelGGL(tile_gateup_kernel<DT_BF16>, dim3(g), dim3(256), 0, s, A, L);
            break;
        }
        default: {
            static DeviceCache c_;
            const int g = per_device(c_, [] { return persistent_grid(tile_gateup_kernel<DT_E4M3>, 0); });
            hipLaunchKernelGGL(tile_gateup_kernel<DT_E4M3>, dim3(g), dim3(256), 0, s, A, L);
            break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_tile_down(int dt, const GArgs& A, const TileList& L, int bm, hipStream_t s) {
    (void)bm;
    switch (dt) {
        case DT_F32: {
            static DeviceCache c_;
            const int g = per_device(c_, [] { return persistent_grid(tile_down_kernel<DT_F32>, 0); });
            hipLaunchKernelGGL(tile_down_kernel<DT_F32>, dim3(g), dim3(256), 0, s, A, L);
            break;
        }
        case DT_BF16: {
            static DeviceCache c_;
            const int g = per_device(c_, [] { return persistent_grid(tile_down_kernel<DT_BF16>, 0); });
            hipLaunchKernelGGL(tile_down_kernel<DT_BF16>, dim3(g), dim3(256), 0, s, A, L);
            break;
        }
        default: {
            static DeviceCache c_;
            const int g = per_device(c_, [] { return persistent_grid(tile_down_kernel<DT_E4M3>, 0); });
            hipLaunchKernelGGL(tile_down_kernel<DT_E4M3>, dim3(g), dim3(256), 0, s, A, L);
            break;
        }
    }
    return hipGetLastError();
}

}  // namespace moe
