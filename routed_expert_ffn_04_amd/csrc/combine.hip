// Combine: out[t] = y_sh[t] + sum_j w[t][j] * y_perm[dest[t*k + j]], fp32
// accumulation in this order ("DeepSeek V3/R1 Inference Efficiency (2)",
// section 2.3.1, operator "Expert: combine reduce").  Memory-bound gather:
// one workgroup per token and 1024-column slab, 4 columns per thread.  The
// expert outputs may arrive as e4m3 with per-1x128 scales (the FP8 combine the
// same page names as the lever from 3300 to 5000 tokens/s per GPU).
#include "common.h"
#include "internal.h"

namespace moe {

// YM: expert outputs y_perm in fp32 (0), bf16 (1) or e4m3 codes with one fp32
// scale per row and 128 columns (2: the fp8 combine); SHB: y_sh in bf16.
template <int YM, bool SHB, bool OB>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm, const float* __restrict__ y_scale,
                                                      const void* __restrict__ y_sh, const int32_t* __restrict__ dest,
                                                      const float* __restrict__ w, int T, int k, int H,
                                                      void* __restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    auto load4 = [&](const void* base, size_t row, bool bf) -> float4 {
        if (bf) {
            const uint2 u = *(const uint2*)((const uint16_t*)base + row * H + c);
            return make_float4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                               bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16));
        }
        return *(const float4*)((const float*)base + row * H + c);
    };
    float4 acc = y_sh ? load4(y_sh, t, SHB) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        const size_t row = (size_t)dest[(size_t)t * k + j];
        float4 v;
        if (YM == 2) {
            // four codes, decoded exactly (v_cvt_pk_f32_fp8), times the block scale
            const int u = *(const int*)((const uint8_t*)y_perm + row * H + c);
            const float sc = y_scale[row * (H / 128) + c / 128];
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(u, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(u, true);
            v = make_float4(lo[0] * sc, lo[1] * sc, hi[0] * sc, hi[1] * sc);
        } else {
            v = load4(y_perm, row, YM == 1);
        }
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

hipError_t launch_combine(const void* y_perm, int y_mode, const float* y_scale, const void* y_sh, int y_sh_bf16,
                          const int32_t* dest, const float* w, int T, int k, int H, void* out, int out_bf16,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    dim3 grid((H / 4 + 255) / 256, T);
#define MOE_COMB(YM, SB, OB)                                                                                   \
    hipLaunchKernelGGL((combine_kernel<YM, SB, OB>), grid, dim3(256), 0, s, y_perm, y_scale, y_sh, dest, w, T, k, \
                       H, out)
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
