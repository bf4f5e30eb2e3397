// Combine: out[t] = y_sh[t] + sum_j w[t][j] * y_perm[dest[t*k + j]], fp32
// accumulation in this order ("DeepSeek V3/R1 Inference Efficiency (2)",
// section 2.3.1, operator "Expert: combine reduce").  Memory-bound gather:
// one workgroup per token and 1024-column slab, 8 columns per thread.  The
// expert outputs may arrive as e4m3 with per-1x128 scales (the FP8 combine the
// same page names as the lever from 3300 to 5000 tokens/s per GPU).
#include "common.h"
#include "internal.h"

namespace moe {

// YM: expert outputs y_perm in fp32 (0), bf16 (1) or e4m3 codes with one fp32
// scale per row and 128 columns (2: the fp8 combine); SHB: y_sh in bf16.
// A thread owns 8 consecutive columns (one 16-byte bf16 load per row, inside
// one 128-column scale block) and issues the loads of up to 8 expert rows
// before it folds them into the accumulator in slot order, so the gathers of
// a token are in flight together.
template <int YM>
struct YRaw;
template <> struct YRaw<0> { float4 a, b; };
template <> struct YRaw<1> { uint4 a; };
template <> struct YRaw<2> { uint2 a; float sc; };

__device__ __forceinline__ void bf16x8_to_f32(const uint4& u, float v[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
}

template <int YM>
__device__ __forceinline__ YRaw<YM> load_y(const void* y, const float* y_scale, size_t row, int H, int c) {
    YRaw<YM> r;
    if constexpr (YM == 0) {
        const float4* p = (const float4*)((const float*)y + row * H + c);
        r.a = p[0];
        r.b = p[1];
    } else if constexpr (YM == 1) {
        r.a = *(const uint4*)((const uint16_t*)y + row * H + c);
    } else {
        r.a = *(const uint2*)((const uint8_t*)y + row * H + c);
        r.sc = y_scale[row * (H / 128) + c / 128];
    }
    return r;
}

template <int YM>
__device__ __forceinline__ void decode_y(const YRaw<YM>& r, float v[8]) {
    if constexpr (YM == 0) {
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    } else if constexpr (YM == 1) {
        bf16x8_to_f32(r.a, v);
    } else {
        // codes decoded exactly (v_cvt_pk_f32_fp8), times the block scale
        const uint32_t w[2] = {r.a.x, r.a.y};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
            v[4 * i] = lo[0] * r.sc;
            v[4 * i + 1] = lo[1] * r.sc;
            v[4 * i + 2] = hi[0] * r.sc;
            v[4 * i + 3] = hi[1] * r.sc;
        }
    }
}

constexpr int kCombCols = 8;      // columns per thread
constexpr int kCombRows = 8;      // expert rows in flight per thread
constexpr int kCombThreads = 128;

template <int YM, bool SHB, bool OB>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const void* __restrict__ y_perm,
                                                               const float* __restrict__ y_scale,
                                                               const void* __restrict__ y_sh,
                                                               const int32_t* __restrict__ dest,
                                                               const float* __restrict__ w, int T, int k, int H,
                                                               void* __restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * kCombThreads + threadIdx.x) * kCombCols;
    if (c >= H) return;
    float acc[kCombCols];
    if (y_sh) {
        if (SHB) {
            bf16x8_to_f32(*(const uint4*)((const uint16_t*)y_sh + (size_t)t * H + c), acc);
        } else {
            const float4* p = (const float4*)((const float*)y_sh + (size_t)t * H + c);
            const float4 a = p[0], b = p[1];
            acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
            acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kCombCols; ++q) acc[q] = 0.f;
    }
    const int32_t* dt = dest + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    for (int j0 = 0; j0 < k; j0 += kCombRows) {
        const int n = min(kCombRows, k - j0);
        YRaw<YM> raw[kCombRows];
#pragma unroll
        for (int jj = 0; jj < kCombRows; ++jj)
            if (jj < n) raw[jj] = load_y<YM>(y_perm, y_scale, (size_t)dt[j0 + jj], H, c);
        // out = y_sh + sum_j w_j * y_j, one fused multiply-add per slot, in slot order
#pragma unroll
        for (int jj = 0; jj < kCombRows; ++jj) {
            if (jj < n) {
                const float wj = wt[j0 + jj];
                float v[kCombCols];
                decode_y<YM>(raw[jj], v);
#pragma unroll
                for (int q = 0; q < kCombCols; ++q) acc[q] = __builtin_fmaf(wj, v[q], acc[q]);
            }
        }
    }
    if (OB) {
        uint4 o;
        o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
        o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
        o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
        o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
        *(uint4*)((uint16_t*)out + (size_t)t * H + c) = o;
    } else {
        float4* p = (float4*)((float*)out + (size_t)t * H + c);
        p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

hipError_t launch_combine(const void* y_perm, int y_mode, const float* y_scale, const void* y_sh, int y_sh_bf16,
                          const int32_t* dest, const float* w, int T, int k, int H, void* out, int out_bf16,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((H / kCombCols + kCombThreads - 1) / kCombThreads, T);
#define MOE_COMB(YM, SB, OB)                                                                                         \
    hipLaunchKernelGGL((combine_kernel<YM, SB, OB>), grid, dim3(kCombThreads), 0, s, y_perm, y_scale, y_sh, dest, w, \
                       T, k, H, out)
#define MOE_COMB_O(YM, SB) \
    do { if (out_bf16) MOE_COMB(YM, SB, true); else MOE_COMB(YM, SB, false); } while (0)
#define MOE_COMB_S(YM) \
    do { if (y_sh_bf16) MOE_COMB_O(YM, true); else MOE_COMB_O(YM, false); } while (0)
    if (y_mode == 2) MOE_COMB_S(2);
    else if (y_mode == 1) MOE_COMB_S(1);
    else MOE_COMB_S(0);
#undef MOE_COMB_S
#undef MOE_COMB_O
#undef MOE_COMB
    return hipGetLastError();
}

}  // namespace moe
