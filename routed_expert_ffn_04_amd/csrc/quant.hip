// Activation quantisation to OCP FP8 E4M3FN with one fp32 scale per row and
// 128-column block: the analogue of the BF16 -> FP8 cast operator of
// "DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1 (the pages name the
// cast; the 1x128 block scale is the reading taken for activations).
//   amax = max |v|;  s = amax / 448 (IEEE fp32 division; 1 if amax == 0);
//   q = e4m3_rne_sat(v / s) (IEEE fp32 division per element).
// Memory-bound: 16 lanes per block, 8 elements per lane (one 16-byte bf16 load).
#include "common.h"
#include "internal.h"

namespace moe {

template <bool XBF16>
__global__ __launch_bounds__(256) void quant_e4m3_kernel(const void* __restrict__ x, int rows, int cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
    const int nb = cols / 128;
    const long blk = (long)blockIdx.x * 16 + threadIdx.x / 16;
    const int sub = threadIdx.x % 16;
    const bool valid = blk < (long)rows * nb;
    const long r = valid ? blk / nb : 0, b = valid ? blk % nb : 0;
    const size_t off = (size_t)r * cols + (size_t)b * 128 + sub * 8;
    float v[8];
    if (valid) {
        if (XBF16) {
            const uint4 u = *(const uint4*)((const uint16_t*)x + off);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            }
        } else {
            const float4 a = *(const float4*)((const float*)x + off);
            const float4 c = *(const float4*)((const float*)x + off + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[4 + i] / s) << (8 * i);
    if (valid) {
        *(uint2*)(q + off) = make_uint2(lo, hi);
        if (sub == 0) scale[(size_t)r * nb + b] = s;
    }
}

// MXFP8 (OCP Microscaling, E4M3 elements with one E8M0 exponent per 32
// consecutive values of a row): the activation format of the MXFP4 expert
// GEMMs.  E from the block's amax (mx_e8m0_for_e4m3); q = e4m3_rne_sat(v *
// 2^(127-E)), where the product is exact.  4 lanes per block, 8 values each.
template <bool XBF16>
__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const void* __restrict__ x, int rows, int cols,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ e8) {
    const int nb = cols / 32;
    const long blk = (long)blockIdx.x * 64 + threadIdx.x / 4;
    const int sub = threadIdx.x % 4;
    const bool valid = blk < (long)rows * nb;
    const long r = valid ? blk / nb : 0, b = valid ? blk % nb : 0;
    const size_t off = (size_t)r * cols + (size_t)b * 32 + sub * 8;
    float v[8];
    if (valid) {
        if (XBF16) {
            const uint4 u = *(const uint4*)((const uint16_t*)x + off);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
                v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            }
        } else {
            const float4 a = *(const float4*)((const float*)x + off);
            const float4 c = *(const float4*)((const float*)x + off + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    const uint32_t E = mx_e8m0_for_e4m3(amax);
    const float f = mx_inv_scale(E);
    const uint32_t lo = f32x4_to_e4m3x4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
    const uint32_t hi = f32x4_to_e4m3x4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
    if (valid) {
        *(uint2*)(q + off) = make_uint2(lo, hi);
        if (sub == 0) e8[(size_t)r * nb + b] = (uint8_t)E;
    }
}

hipError_t launch_quant_mxfp8(const void* x, int x_bf16, int rows, int cols, uint8_t* q, uint8_t* e8,
                              hipStream_t s) {
    const long nblk = (long)rows * (cols / 32);
    if (nblk == 0) return hipSuccess;
    dim3 grid((unsigned)((nblk + 63) / 64));
    if (x_bf16)
        hipLaunchKernelGGL(quant_mxfp8_kernel<true>, grid, dim3(256), 0, s, x, rows, cols, q, e8);
    else
        hipLaunchKernelGGL(quant_mxfp8_kernel<false>, grid, dim3(256), 0, s, x, rows, cols, q, e8);
    return hipGetLastError();
}

hipError_t launch_quant_e4m3(const void* x, int x_bf16, int rows, int cols, uint8_t* q, float* scale,
                             hipStream_t s) {
    const long nblk = (long)rows * (cols / 128);
    if (nblk == 0) return hipSuccess;
    dim3 grid((unsigned)((nblk + 15) / 16));
    if (x_bf16)
        hipLaunchKernelGGL(quant_e4m3_kernel<true>, grid, dim3(256), 0, s, x, rows, cols, q, scale);
    else
        hipLaunchKernelGGL(quant_e4m3_kernel<false>, grid, dim3(256), 0, s, x, rows, cols, q, scale);
    return hipGetLastError();
}

}  // namespace moe
