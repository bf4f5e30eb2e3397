// Router: fp32 logits with a fixed fused-multiply-add order, then top-k and
// renormalised weights ("How DeepSeek inference works", section "What does
// DeepSeek inference actually do per token?"; "DeepSeek V3/R1 Inference
// Efficiency (2)", section 2.3.1, operator "Gate: router gate").
//
// The expert ids must be identical to a plain CPU evaluation, so every logit
// is ONE fp32 chain: acc = fma(x[t][h], Wr[h][e], acc) for h ascending.  This
// rules out matrix cores and any split of the h range; the kernel is a
// register-tiled SIMT product in which each thread owns RT x RE logits and
// walks h in order.  Work per logit is H FMAs; the whole router is T*E*H FMAs
// on the fp32 vector units (no contraction flags: built with
// -ffp-contract=off, FMAs are explicit).
#include "common.h"
#include "internal.h"

namespace moe {

// Tile: TT = NY*RT tokens x TE = NX*RE experts per workgroup of NX x NY
// threads, each thread owning RT x RE logits.  h is consumed in chunks of KC: while the
// chunk in LDS is being used, the next one is already loaded into registers,
// and it is written to the other LDS buffer afterwards (one barrier per
// chunk).  Loads are 16-byte vectors; rows and columns past T and E are
// clamped to valid ones (their logits are computed and discarded), so the
// staging has no branches.  x is stored transposed ([h][token]) with
// consecutive threads on consecutive tokens (conflict-free).
template <int RT, int RE, int KC, int NX, int NY, bool XBF16, bool WVEC>
__global__ __launch_bounds__(NX * NY) void router_logits_kernel(const void* __restrict__ xv, int T, int H,
                                                                const float* __restrict__ wr,
                                                                const float* __restrict__ bias, int E,
                                                                float* __restrict__ logits) {
    constexpr int NT = NX * NY;                      // threads
    constexpr int TT = NY * RT, TE = NX * RE;
    constexpr int NXV = TT * KC / 8 / NT;           // 8-element x vectors per thread
    constexpr int NWV = KC * TE / 4 / NT;           // 4-element W vectors per thread
    static_assert(NXV * 8 * NT == TT * KC && NWV * 4 * NT == KC * TE, "tile");
    __shared__ float xs[2][KC][TT];
    __shared__ __attribute__((aligned(16))) float wsm[2][KC][TE];
    const int tid = threadIdx.x, tx = tid % NX, ty = tid / NX;
    const int t0 = blockIdx.y * TT, e0 = blockIdx.x * TE;

    float rx[NXV][8];
    f32x4 rw[NWV];
    auto fetch = [&](int h0) {
#pragma unroll
        for (int v = 0; v < NXV; ++v) {
            const int idx = tid + v * NT, r = idx % TT, cg = idx / TT;
            const size_t off = (size_t)min(t0 + r, T - 1) * H + h0 + cg * 8;
            if (XBF16) {
                const uint4 u = *(const uint4*)((const uint16_t*)xv + off);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    rx[v][2 * q] = bf16_bits_to_f32(w4[q] & 0xFFFFu);
                    rx[v][2 * q + 1] = bf16_bits_to_f32(w4[q] >> 16);
                }
            } else {
                const float4 a = *(const float4*)((const float*)xv + off);
                const float4 b = *(const float4*)((const float*)xv + off + 4);
                rx[v][0] = a.x; rx[v][1] = a.y; rx[v][2] = a.z; rx[v][3] = a.w;
                rx[v][4] = b.x; rx[v][5] = b.y; rx[v][6] = b.z; rx[v][7] = b.w;
            }
        }
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            const int idx = tid + v * NT, c = idx / (TE / 4), q4 = idx % (TE / 4);
            const float* row = wr + (size_t)(h0 + c) * E;
            if (WVEC) {
                rw[v] = *(const f32x4*)(row + min(e0 + q4 * 4, E - 4));
            } else {
                const int e = e0 + q4 * 4;
                rw[v] = f32x4{row[min(e, E - 1)], row[min(e + 1, E - 1)], row[min(e + 2, E - 1)],
                              row[min(e + 3, E - 1)]};
            }
        }
    };
    auto stash = [&](int b) {
#pragma unroll
        for (int v = 0; v < NXV; ++v) {
            const int idx = tid + v * NT, r = idx % TT, cg = idx / TT;
#pragma unroll
            for (int q = 0; q < 8; ++q) xs[b][cg * 8 + q][r] = rx[v][q];
        }
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            const int idx = tid + v * NT, c = idx / (TE / 4), q4 = idx % (TE / 4);
            *(f32x4*)&wsm[b][c][q4 * 4] = rw[v];
        }
    };

    float acc[RT][RE];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) acc[i][j] = 0.0f;

    const int nch = H / KC;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int b = ch & 1;
        if (ch + 1 < nch) fetch((ch + 1) * KC);
#pragma unroll 8
        for (int c = 0; c < KC; ++c) {
            float a[RT], w[RE];
#pragma unroll
            for (int i = 0; i < RT; ++i) a[i] = xs[b][c][ty * RT + i];
#pragma unroll
            for (int j = 0; j < RE; ++j) w[j] = wsm[b][c][tx * RE + j];
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < RE; ++j) acc[i][j] = __builtin_fmaf(a[i], w[j], acc[i][j]);
        }
        if (ch + 1 < nch) stash(b ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = t0 + ty * RT + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < RE; ++j) {
            const int e = e0 + tx * RE + j;
            if (e >= E) continue;
            float l = acc[i][j] + (bias ? bias[e] : 0.0f);
            l = l + 0.0f;   // -0 -> +0
            logits[(size_t)t * E + e] = l;
        }
    }
}

// One logit per thread (small batches): the same chains and chunking, with
// the LDS tiles stored h-contiguous per token and per expert ([TT][KC] and
// [TE][KC], rows padded by 4 floats so that the NY token rows and NX expert
// rows of a wave fall in distinct banks), so a thread reads four consecutive
// h values of its x row and W column with one 16-byte load each.
template <int KC, int NX, int NY, bool XBF16, bool WVEC>
__global__ __launch_bounds__(NX * NY) void router_chain_kernel(const void* __restrict__ xv, int T, int H,
                                                               const float* __restrict__ wr,
                                                               const float* __restrict__ bias, int E,
                                                               float* __restrict__ logits) {
    constexpr int NT = NX * NY, TT = NY, TE = NX, KP = KC + 4;
    constexpr int NXV = TT * KC / 8 / NT;           // 8-element x vectors per thread
    constexpr int NWV = KC * TE / 4 / NT;           // 4-element W vectors per thread
    static_assert(NXV * 8 * NT == TT * KC && NWV * 4 * NT == KC * TE, "tile");
    __shared__ __attribute__((aligned(16))) float xs[2][TT][KP];
    __shared__ __attribute__((aligned(16))) float wsm[2][TE][KP];
    const int tid = threadIdx.x, tx = tid % NX, ty = tid / NX;
    const int t0 = blockIdx.y * TT, e0 = blockIdx.x * TE;

    float rx[NXV][8];
    f32x4 rw[NWV];
    auto fetch = [&](int h0) {
#pragma unroll
        for (int v = 0; v < NXV; ++v) {
            const int idx = tid + v * NT, r = idx % TT, cg = idx / TT;
            const size_t off = (size_t)min(t0 + r, T - 1) * H + h0 + cg * 8;
            if (XBF16) {
                const uint4 u = *(const uint4*)((const uint16_t*)xv + off);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    rx[v][2 * q] = bf16_bits_to_f32(w4[q] & 0xFFFFu);
                    rx[v][2 * q + 1] = bf16_bits_to_f32(w4[q] >> 16);
                }
            } else {
                const float4 a = *(const float4*)((const float*)xv + off);
                const float4 b = *(const float4*)((const float*)xv + off + 4);
                rx[v][0] = a.x; rx[v][1] = a.y; rx[v][2] = a.z; rx[v][3] = a.w;
                rx[v][4] = b.x; rx[v][5] = b.y; rx[v][6] = b.z; rx[v][7] = b.w;
            }
        }
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            const int idx = tid + v * NT, c = idx / (TE / 4), q4 = idx % (TE / 4);
            const float* row = wr + (size_t)(h0 + c) * E;
            if (WVEC) {
                rw[v] = *(const f32x4*)(row + min(e0 + q4 * 4, E - 4));
            } else {
                const int e = e0 + q4 * 4;
                rw[v] = f32x4{row[min(e, E - 1)], row[min(e + 1, E - 1)], row[min(e + 2, E - 1)],
                              row[min(e + 3, E - 1)]};
            }
        }
    };
    auto stash = [&](int b) {
#pragma unroll
        for (int v = 0; v < NXV; ++v) {
            const int idx = tid + v * NT, r = idx % TT, cg = idx / TT;
            *(f32x4*)&xs[b][r][cg * 8] = f32x4{rx[v][0], rx[v][1], rx[v][2], rx[v][3]};
            *(f32x4*)&xs[b][r][cg * 8 + 4] = f32x4{rx[v][4], rx[v][5], rx[v][6], rx[v][7]};
        }
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            const int idx = tid + v * NT, c = idx / (TE / 4), q4 = idx % (TE / 4);
#pragma unroll
            for (int m = 0; m < 4; ++m) wsm[b][q4 * 4 + m][c] = rw[v][m];
        }
    };

    float acc = 0.0f;
    const int nch = H / KC;
    fetch(0);
    stash(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int b = ch & 1;
        if (ch + 1 < nch) fetch((ch + 1) * KC);
#pragma unroll 8
        for (int c = 0; c < KC; c += 4) {
            const f32x4 a = *(const f32x4*)&xs[b][ty][c];
            const f32x4 w = *(const f32x4*)&wsm[b][tx][c];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_fmaf(a[q], w[q], acc);
        }
        if (ch + 1 < nch) stash(b ^ 1);
        __syncthreads();
    }
    const int t = t0 + ty, e = e0 + tx;
    if (t < T && e < E) {
        float l = acc + (bias ? bias[e] : 0.0f);
        l = l + 0.0f;   // -0 -> +0
        logits[(size_t)t * E + e] = l;
    }
}

template <int KC, int NX, int NY>
static hipError_t launch_chain(const void* x, int xb, int T, int H, const float* wr, const float* bias, int E,
                               float* logits, hipStream_t s) {
    dim3 grid((E + NX - 1) / NX, (T + NY - 1) / NY);
    const bool wvec = E % 4 == 0 && ((uintptr_t)wr & 15) == 0;
#define MOE_RC(XB, WV)                                                                                           \
    hipLaunchKernelGGL((router_chain_kernel<KC, NX, NY, XB, WV>), grid, dim3(NX * NY), 0, s, x, T, H, wr, bias, E, \
                       logits)
    if (xb) { if (wvec) MOE_RC(true, true); else MOE_RC(true, false); }
    else { if (wvec) MOE_RC(false, true); else MOE_RC(false, false); }
#undef MOE_RC
    return hipGetLastError();
}

template <int RT, int RE, int KC, int NX = 16, int NY = 16>
static hipError_t launch_rl(const void* x, int xb, int T, int H, const float* wr, const float* bias,
                            int E, float* logits, hipStream_t s) {
    dim3 grid((E + NX * RE - 1) / (NX * RE), (T + NY * RT - 1) / (NY * RT));
    const bool wvec = E % 4 == 0 && ((uintptr_t)wr & 15) == 0;
#define MOE_RL(XB, WV)                                                                                          \
    hipLaunchKernelGGL((router_logits_kernel<RT, RE, KC, NX, NY, XB, WV>), grid, dim3(NX * NY), 0, s, x, T, H, wr, \
                       bias, E, logits)
    if (xb) { if (wvec) MOE_RL(true, true); else MOE_RL(true, false); }
    else { if (wvec) MOE_RL(false, true); else MOE_RL(false, false); }
#undef MOE_RL
    return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, int x_bf16, int T, int H, const float* wr,
                                const float* bias, int E, float* logits, hipStream_t s) {
    // Large batches: big register tiles (FMA:LDS ratio).  Small batches: one
    // logit per thread so that enough chains run side by side, one-wave
    // workgroups (8 x 8 logits) so that the few chains spread over every CU
    // (T = 128, E = 256: 512 workgroups), and the longest h chunk that divides
    // H, so that fewer chunk barriers interrupt the chains (T = 128, H = 7168:
    // 105 us with 16 x 16 tiles and h-strided LDS reads, 70 us with the chain
    // kernel at 128-long chunks, 52 us at 512).  H is a multiple of 128.
    const long chains = (long)T * E;
    if (chains >= (1L << 21) && E >= 64) return launch_rl<8, 4, 32>(x, x_bf16, T, H, wr, bias, E, logits, s);
    if (chains >= (1L << 18)) return launch_rl<4, 2, 64>(x, x_bf16, T, H, wr, bias, E, logits, s);
    if (H % 512 == 0) return launch_chain<512, 8, 8>(x, x_bf16, T, H, wr, bias, E, logits, s);
    if (H % 256 == 0) return launch_chain<256, 8, 8>(x, x_bf16, T, H, wr, bias, E, logits, s);
    return launch_chain<128, 8, 8>(x, x_bf16, T, H, wr, bias, E, logits, s);
}

// ---- top-k + weights: one wave per token ----------------------------------
// Each lane holds the logits of experts lane, lane+64, ...; a candidate is the
// 64-bit key (order-preserving logit bits << 32 | (0xFFFFFFFF - e)), so the
// wave maximum is the largest logit and, among equal logits, the lowest e.
constexpr int kTopkWaves = 4;

// NS = logits per lane (E <= 64 * NS)
template <int NS>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                          int k, int sigmoid, int32_t* __restrict__ ids,
                                                          float* __restrict__ wout) {
    __shared__ int32_t sel[kTopkWaves][1024];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kTopkWaves + wave;
    const bool valid = t < T;          // no early return: the barrier below needs every wave
    const float* lt = logits + (size_t)(valid ? t : 0) * E;
    uint64_t key[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int e = s * kWave + lane;
        key[s] = 0;
        if (valid && e < E) key[s] = ((uint64_t)f32_order_key(lt[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
    for (int j = 0; j < (valid ? k : 0); ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int s = 0; s < NS; ++s) best = key[s] > best ? key[s] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        if ((e & (kWave - 1)) == lane) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                if (s == (e >> 6)) key[s] = 0;
        }
        if (lane == 0) sel[wave][j] = e;
    }
    __syncthreads();
    if (!valid) return;
    // weights in double: sigmoid scores or exp(l - l_max), renormalised
    const double l0 = (double)lt[sel[wave][0]];
    double part = 0.0;
    for (int j = lane; j < k; j += kWave) {
        const double l = (double)lt[sel[wave][j]];
        part += sigmoid ? 1.0 / (1.0 + exp(-l)) : exp(l - l0);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m, kWave);
    for (int j = lane; j < k; j += kWave) {
        const int e = sel[wave][j];
        const double l = (double)lt[e];
        const double sc = sigmoid ? 1.0 / (1.0 + exp(-l)) : exp(l - l0);
        ids[(size_t)t * k + j] = e;
        wout[(size_t)t * k + j] = (float)(sc / part);
    }
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int sigmoid, int32_t* ids,
                              float* w, hipStream_t s) {
    dim3 grid((T + kTopkWaves - 1) / kTopkWaves);
#define MOE_TOPK(NSV) hipLaunchKernelGGL(router_topk_kernel<NSV>, grid, dim3(256), 0, s, logits, T, E, k, sigmoid, ids, w)
    if (E <= 64) MOE_TOPK(1);
    else if (E <= 128) MOE_TOPK(2);
    else if (E <= 256) MOE_TOPK(4);
    else if (E <= 512) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

}  // namespace moe
