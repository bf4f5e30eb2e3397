// Combine: out[t] = y_sh[t] + sum_j w[t][j] * y_perm[dest[t*k + j]], fp32
// accumulation in this order ("DeepSeek V3/R1 Inference Efficiency (2)",
// section 2.3.1, operator "Expert: combine reduce").  Memory-bound gather:
// one workgroup per token and 1024-column slab, 4 columns per thread.
#include "common.h"
#include "internal.h"

namespace moe {

template <bool YB, bool OB>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm, const void* __restrict__ y_sh,
                                                      const int32_t* __restrict__ dest, const float* __restrict__ w,
                                                      int T, int k, int H, void* __restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    auto load4 = [&](const void* base, size_t row) -> float4 {
        if (YB) {
            const uint2 u = *(const uint2*)((const uint16_t*)base + row * H + c);
            return make_float4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                               bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16));
        }
        return *(const float4*)((const float*)base + row * H + c);
    };
    float4 acc = y_sh ? load4(y_sh, t) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const float4 v = load4(y_perm, (size_t)dest[(size_t)t * k + j]);
        acc.x = __builtin_fmaf(wj, v.x, acc.x);
        acc.y = __builtin_fmaf(wj, v.y, acc.y);
        acc.z = __builtin_fmaf(wj, v.z, acc.z);
        acc.w = __builtin_fmaf(wj, v.w, acc.w);
    }
    if (OB) {
        const uint32_t lo = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
        const uint32_t hi = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
        *(uint2*)((uint16_t*)out + (size_t)t * H + c) = make_uint2(lo, hi);
    } else {
        *(float4*)((float*)out + (size_t)t * H + c) = acc;
    }
}

hipError_t launch_combine(const void* y_perm, const void* y_sh, int y_bf16, const int32_t* dest, const float* w,
                          int T, int k, int H, void* out, int out_bf16, hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((H / 4 + 255) / 256, T);
#define MOE_COMB(YB, OB) hipLaunchKernelGGL((combine_kernel<YB, OB>), grid, dim3(256), 0, s, y_perm, y_sh, dest, w, T, k, H, out)
    if (y_bf16 && out_bf16) MOE_COMB(true, true);
    else if (y_bf16) MOE_COMB(true, false);
    else if (out_bf16) MOE_COMB(false, true);
    else MOE_COMB(false, false);
#undef MOE_COMB
    return hipGetLastError();
}

}  // namespace moe
