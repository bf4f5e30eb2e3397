// Grouped expert FFN, weight-streaming kernels for groups of few rows (bf16).
//
// In the small-m regime ("DeepSeek V3/R1 Inference Efficiency (2)", section
// 2.4.1, the decode-time routed expert GEMMs with a handful of rows per expert)
// the work is bound by reading every weight of every touched expert once.
// These kernels therefore keep weights out of LDS: each wave loads its weight
// fragments from HBM straight into registers in the MFMA operand layout
// (lane = output column, 8 consecutive k per lane, 16-byte loads), keeps P
// k-steps of loads in flight, and reads the few activation rows from L2.
// The four waves of a workgroup split K; their partial sums meet in LDS, where
// the gate/up epilogue applies SwiGLU and rounds h to bf16.
//
// Tile: MB*16 rows x TN output columns x all of K.  Rows past the group's end
// re-read its last row (no masked loads, no branches in the k loop) and are
// never stored.
#include "gffn_common.h"

namespace moe {

constexpr int kP = 4;                 // k-steps of loads in flight per wave (64-row tiles)
constexpr int kPD = 8;                // the same for the 16-row down tiles (8: 0.5% faster than 4 at T = 128)
// 16-row gate/up tiles (whole K per wave): k-steps in flight and 16-column
// blocks per wave.  On the T = 128 decode layer, one block with 16 k-steps in
// flight (two 1 KiB weight fragments per k-step and wave, two workgroups per
// CU) beat two blocks with 8 (4.06 -> 3.87 ms of grouped FFN), which beat two
// with 4 (4.08 ms) and 2 (4.15 ms).  H not a multiple of 512: 4 in flight.
constexpr int kPG = 16;
constexpr int kNBG = 1;
constexpr int kNB = 2;                // 16-column blocks per wave
// 64-row gate/up tiles split K over the four waves.
constexpr int kKsGateup = 4;

// Weight loads use the default cache policy: measured on MI355X, the
// non-temporal hint made the streaming kernels ~15% slower.
__device__ __forceinline__ bf16x8 ldw(const uint16_t* p) { return *(const bf16x8*)p; }

__device__ __forceinline__ bf16x8 lda(const uint16_t* p) { return *(const bf16x8*)p; }

// ---------------------------------------------------------------- gate / up
template <int MB, int KS, int P, int NB>
__global__ __launch_bounds__(256) void stream_gateup_kernel(GArgs A, TileList L) {
    constexpr int NW = 4 / KS;                 // waves along N
    constexpr int TN = NW * NB * 16;          // h columns per tile
    constexpr int RS = 2 * TN + 1;             // LDS row stride (floats)
    const int H = A.H, I = A.I;
    const int ntn = I / TN;
    const int nsteps = H / 32 / KS;            // k-steps of 32 per wave

    __shared__ float red[KS][16 * MB][RS];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int kw = wave % KS, nw = wave / KS;

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        const int t = (int)it.t;
        __syncthreads();   // the previous tile's reduction is done with `red`
        const int2 tc = tile_coords<MB == 1>(L, t, ntn);
        const int2 tl = L.entries[tc.x];
        const GroupInfo gi = group_info(A, tl.x);
        const int m0 = tl.y;
        const int nt0 = tc.y * TN;
        const int n0 = nt0 + nw * NB * 16;
        const Bank& bk = gi.shared ? A.shared : A.routed;
        const int kb = kw * nsteps * 32 + (lane / 16) * 8;

        // Rows past the group's end read the last valid row instead: MFMA rows
        // do not mix, and those rows are never stored.
        const uint16_t* ap[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int r = min(m0 + i * 16 + lane % 16, gi.m - 1);
            int ar;
            const uint16_t* base;
            if (gi.shared) {
                ar = r;
                base = (const uint16_t*)A.a_sh;
            } else {
                const int pp = gi.p0 + r;
                ar = A.src ? A.src[pp] / A.src_div : pp;
                base = (const uint16_t*)A.a;
            }
            ap[i] = base + (size_t)ar * H + kb;
        }
        const uint16_t* gp[NB];
        const uint16_t* up[NB];
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            const size_t row = (size_t)gi.e * I + n0 + c * 16 + lane % 16;
            gp[c] = (const uint16_t*)bk.wg + row * H + kb;
            up[c] = (const uint16_t*)bk.wu + row * H + kb;
        }

        f32x4 accg[MB][NB], accu[MB][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < NB; ++c) accg[i][c] = accu[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ring of P k-steps in flight; nsteps is a multiple of P, the body
        // is straight-line so the loads of later steps stay outstanding
        bf16x8 ra[P][MB], rg[P][NB], ru[P][NB];
        auto load = [&](int p, int step) {
#pragma unroll
            for (int c = 0; c < NB; ++c) {
                rg[p][c] = ldw(gp[c] + step * 32);
                ru[p][c] = ldw(up[c] + step * 32);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) ra[p][i] = lda(ap[i] + step * 32);
        };
        auto mma = [&](int p) {
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    accg[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[p][i], rg[p][c], accg[i][c], 0, 0, 0);
                    accu[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[p][i], ru[p][c], accu[i][c], 0, 0, 0);
                }
        };
#pragma unroll
        for (int p = 0; p < P; ++p) load(p, p);
        for (int s0 = 0; s0 < nsteps - P; s0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                mma(p);
                load(p, s0 + P + p);
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) mma(p);

        // partial sums -> LDS; row = i*16 + 4*(lane/16) + q, col = (n0 - nt0) + c*16 + lane%16
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < NB; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = i * 16 + 4 * (lane / 16) + q;
                    const int col = nw * NB * 16 + c * 16 + lane % 16;
                    red[kw][row][col] = accg[i][c][q];
                    red[kw][row][TN + col] = accu[i][c][q];
                }
        __syncthreads();
        for (int e = tid; e < 16 * MB * TN; e += 256) {
            const int row = e / TN, col = e % TN;
            const int r = m0 + row;
            if (r >= gi.m) continue;
            float g = 0.f, u = 0.f;
#pragma unroll
            for (int w = 0; w < KS; ++w) {
                g += red[w][row][col];
                u += red[w][row][TN + col];
            }
            const int hr = h_row(A, gi, r);
            ((uint16_t*)A.h)[(size_t)hr * I + nt0 + col] = (uint16_t)f32_to_bf16_bits(silu_mul(g, u));
        }
    }
}

// ---------------------------------------------------------------- down
template <int MB, int KS, int P>
__global__ __launch_bounds__(256) void stream_down_kernel(GArgs A, TileList L) {
    constexpr int NW = 4 / KS;
    constexpr int TN = NW * kNB * 16;          // output (H) columns per tile
    constexpr int RS = TN + 1;
    const int H = A.H, I = A.I;
    const int ntn = H / TN;
    const int nsteps = I / 32 / KS;

    __shared__ float red[KS][16 * MB][RS];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int kw = wave % KS, nw = wave / KS;

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        const int t = (int)it.t;
        __syncthreads();   // the previous tile's reduction is done with `red`
        const int2 tc = tile_coords<MB == 1>(L, t, ntn);
        const int2 tl = L.entries[tc.x];
        const GroupInfo gi = group_info(A, tl.x);
        const int m0 = tl.y;
        const int nt0 = tc.y * TN;
        const int n0 = nt0 + nw * kNB * 16;
        const Bank& bk = gi.shared ? A.shared : A.routed;
        const int kb = kw * nsteps * 32 + (lane / 16) * 8;

        const uint16_t* ap[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int r = min(m0 + i * 16 + lane % 16, gi.m - 1);   // see gate/up
            ap[i] = (const uint16_t*)A.h + (size_t)h_row(A, gi, r) * I + kb;
        }
        const uint16_t* dp[kNB];
#pragma unroll
        for (int c = 0; c < kNB; ++c)
            dp[c] = (const uint16_t*)bk.wd + ((size_t)gi.e * H + n0 + c * 16 + lane % 16) * I + kb;

        f32x4 acc[MB][kNB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        bf16x8 ra[P][MB], rd[P][kNB];
        auto load = [&](int p, int step) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) rd[p][c] = ldw(dp[c] + step * 32);
#pragma unroll
            for (int i = 0; i < MB; ++i) ra[p][i] = lda(ap[i] + step * 32);
        };
        auto mma = [&](int p) {
#pragma unroll
            for (int c = 0; c < kNB; ++c)
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[p][i], rd[p][c], acc[i][c], 0, 0, 0);
        };
#pragma unroll
        for (int p = 0; p < P; ++p) load(p, p);
        for (int s0 = 0; s0 < nsteps - P; s0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                mma(p);
                load(p, s0 + P + p);
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) mma(p);

#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[kw][i * 16 + 4 * (lane / 16) + q][nw * kNB * 16 + c * 16 + lane % 16] = acc[i][c][q];
        __syncthreads();
        void* yb = gi.shared ? A.y_sh : A.y;
        for (int e = tid; e < 16 * MB * TN; e += 256) {
            const int row = e / TN, col = e % TN;
            const int r = m0 + row;
            if (r >= gi.m) continue;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < KS; ++w) v += red[w][row][col];
            const size_t yr = gi.shared ? (size_t)r : (size_t)(gi.p0 + r);
            if (gi.shared ? A.y_sh_bf16 : A.y_bf16) ((uint16_t*)yb)[yr * H + nt0 + col] = (uint16_t)f32_to_bf16_bits(v);
            else ((float*)yb)[yr * H + nt0 + col] = v;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <class K>
static int persistent_grid(K kernel) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    return per_cu * device_cu_count();
}

// Tiles of 16 rows: each wave streams whole weight rows (all of K) for its
// kNBG * 16 h columns.  Measured on the T = 128 decode batch, this is about 1% faster
// per layer than splitting K over the four waves, which reads every weight
// row in four pieces.  Tiles of 64 rows split K over the 4 waves when every
// wave still gets a multiple of kP k-steps of 32; otherwise each wave covers
// all of K (K is a multiple of 128, so K/32 is a multiple of 4; kP must
// divide it).
#define MOE_STREAM_LAUNCH(KERNEL, ...)                                               \
    do {                                                                             \
        static DeviceCache cache_;                                                   \
        const int g = per_device(cache_, [] { return persistent_grid(KERNEL<__VA_ARGS__>); }); \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__>), dim3(g), dim3(256), 0, s, A, L);   \
    } while (0)

hipError_t launch_stream_gateup(int mb, const GArgs& A, const TileList& L, hipStream_t s) {
    const bool split = kKsGateup == 4 && A.H % (32 * 4 * kP) == 0;
    if (mb == 1 && A.H % (32 * kPG) == 0) MOE_STREAM_LAUNCH(stream_gateup_kernel, 1, 1, kPG, kNBG);
    else if (mb == 1) MOE_STREAM_LAUNCH(stream_gateup_kernel, 1, 1, kP, kNBG);
    else if (split) MOE_STREAM_LAUNCH(stream_gateup_kernel, 4, 4, kP, kNB);
    else MOE_STREAM_LAUNCH(stream_gateup_kernel, 4, 1, kP, kNB);
    return hipGetLastError();
}

// The down projection's K (= I) is short, so each wave covers all of it and
// a tile is 128 output columns wide.
hipError_t launch_stream_down(int mb, const GArgs& A, const TileList& L, hipStream_t s) {
    static_assert(kP == 1 || kP == 2 || kP == 4, "kP must divide K/32 for every K multiple of 128");
    if (mb == 1 && A.I % (32 * kPD) == 0) MOE_STREAM_LAUNCH(stream_down_kernel, 1, 1, kPD);
    else if (mb == 1) MOE_STREAM_LAUNCH(stream_down_kernel, 1, 1, kP);
    else MOE_STREAM_LAUNCH(stream_down_kernel, 4, 1, kP);
    return hipGetLastError();
}
#undef MOE_STREAM_LAUNCH

}  // namespace moe
