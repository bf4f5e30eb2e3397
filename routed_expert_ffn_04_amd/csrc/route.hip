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

constexpr int kRouterKC = 32;   // h values staged in LDS per step

template <int RT, int RE, bool XBF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ xv, int T, int H,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int E,
                                                            float* __restrict__ logits) {
    constexpr int TT = 16 * RT, TE = 16 * RE, KC = kRouterKC;
    __shared__ float xs[KC][TT];
    __shared__ float wsm[KC][TE];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int t0 = blockIdx.y * TT, e0 = blockIdx.x * TE;

    float acc[RT][RE];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < RE; ++j) acc[i][j] = 0.0f;

    for (int h0 = 0; h0 < H; h0 += KC) {
        // stage x[t0 .. t0+TT)[h0 .. h0+KC) transposed, coalesced along h
        for (int i = tid; i < TT * KC; i += 256) {
            const int r = i / KC, c = i % KC, t = t0 + r;
            float v = 0.0f;
            if (t < T) {
                const size_t off = (size_t)t * H + h0 + c;
                v = XBF16 ? bf16_bits_to_f32(((const uint16_t*)xv)[off]) : ((const float*)xv)[off];
            }
            xs[c][r] = v;
        }
        // stage Wr[h0 .. h0+KC)[e0 .. e0+TE), coalesced along e
        for (int i = tid; i < KC * TE; i += 256) {
            const int c = i / TE, q = i % TE, e = e0 + q;
            wsm[c][q] = (e < E) ? wr[(size_t)(h0 + c) * E + e] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int c = 0; c < KC; ++c) {
            float a[RT], b[RE];
#pragma unroll
            for (int i = 0; i < RT; ++i) a[i] = xs[c][ty * RT + i];
#pragma unroll
            for (int j = 0; j < RE; ++j) b[j] = wsm[c][tx * RE + j];
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < RE; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
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

template <int RT, int RE>
static hipError_t launch_rl(const void* x, int xb, int T, int H, const float* wr, const float* bias,
                            int E, float* logits, hipStream_t s) {
    dim3 grid((E + 16 * RE - 1) / (16 * RE), (T + 16 * RT - 1) / (16 * RT));
    if (xb)
        hipLaunchKernelGGL((router_logits_kernel<RT, RE, true>), grid, dim3(256), 0, s, x, T, H, wr, bias, E, logits);
    else
        hipLaunchKernelGGL((router_logits_kernel<RT, RE, false>), grid, dim3(256), 0, s, x, T, H, wr, bias, E, logits);
    return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, int x_bf16, int T, int H, const float* wr,
                                const float* bias, int E, float* logits, hipStream_t s) {
    // Larger register tiles raise FMA:LDS ratio; small T keeps one logit per
    // thread so that enough chains run in parallel.
    const long chains = (long)T * E;
    if (chains >= (1L << 21) && E >= 64) return launch_rl<8, 4>(x, x_bf16, T, H, wr, bias, E, logits, s);
    if (chains >= (1L << 18)) return launch_rl<4, 2>(x, x_bf16, T, H, wr, bias, E, logits, s);
    return launch_rl<1, 1>(x, x_bf16, T, H, wr, bias, E, logits, s);
}

// ---- top-k + weights: one wave per token ----------------------------------
// Each lane holds the logits of experts lane, lane+64, ...; a candidate is the
// 64-bit key (order-preserving logit bits << 32 | (0xFFFFFFFF - e)), so the
// wave maximum is the largest logit and, among equal logits, the lowest e.
constexpr int kTopkWaves = 4;
constexpr int kMaxSlots = 16;   // E <= 1024

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                          int k, int sigmoid, int32_t* __restrict__ ids,
                                                          float* __restrict__ wout) {
    __shared__ int32_t sel[kTopkWaves][1024];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kTopkWaves + wave;
    const bool valid = t < T;          // no early return: the barrier below needs every wave
    const float* lt = logits + (size_t)(valid ? t : 0) * E;
    uint64_t key[kMaxSlots];
#pragma unroll
    for (int s = 0; s < kMaxSlots; ++s) {
        const int e = s * kWave + lane;
        key[s] = 0;
        if (valid && e < E) key[s] = ((uint64_t)f32_order_key(lt[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
    for (int j = 0; j < (valid ? k : 0); ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int s = 0; s < kMaxSlots; ++s) best = key[s] > best ? key[s] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        if ((e & (kWave - 1)) == lane) {
#pragma unroll
            for (int s = 0; s < kMaxSlots; ++s)
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
    hipLaunchKernelGGL(router_topk_kernel, grid, dim3(256), 0, s, logits, T, E, k, sigmoid, ids, w);
    return hipGetLastError();
}

}  // namespace moe
