// Accuracy of the gfx950 fp8 block MFMA (v_mfma_scale_f32_16x16x128_f8f6f4,
// unit scales) against exact dot products: 4096 random 16x16x128 products of
// e4m3 operands (every finite code equally likely), each output compared with
// the fp64 sum of its 128 exact products.  Prints, for the output lane layout
// (lane l, element q) -> (row 4 (l / 16) + q, column l % 16) and its
// transpose, the largest and mean |error| / sum |products| and the share of
// outputs equal to the fp32 rounding of the exact sum.  The first layout is
// the instruction's; its figures bound what the grouped FFN's fp8 sums can
// differ from the oracle's.
//
// build: hipcc --offload-arch=gfx950 -O2 -Xclang -target-feature -Xclang -packed-fp32-ops \
//          measure/mfma_fp8_accuracy.hip -o measure/mfma_fp8_accuracy
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include <cmath>
#include <vector>
#include <random>
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A: [NT][16][128] bytes, B: [NT][16][128] bytes, D: [NT][64 lanes][4]
__global__ void k(const uint8_t* A, const uint8_t* B, float* D, int NT) {
    int t = blockIdx.x; if (t >= NT) return;
    int l = threadIdx.x;
    const uint8_t* a = A + (size_t)t * 2048 + (l % 16) * 128 + (l / 16) * 32;
    const uint8_t* b = B + (size_t)t * 2048 + (l % 16) * 128 + (l / 16) * 32;
    i32x8 va, vb;
    for (int i = 0; i < 8; ++i) { va[i] = ((const int*)a)[i]; vb[i] = ((const int*)b)[i]; }
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, c, 0, 0, 0, 127, 0, 127);
    for (int q = 0; q < 4; ++q) D[((size_t)t * 64 + l) * 4 + q] = c[q];
}

static double e4m3(uint8_t v) {
    int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
    double r = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
    return s ? -r : r;
}

int main() {
    const int NT = 4096;
    std::vector<uint8_t> A(NT * 2048), B(NT * 2048);
    std::mt19937 g(1);
    for (auto& v : A) { do v = g() & 0xff; while ((v & 0x7f) == 0x7f); }
    for (auto& v : B) { do v = g() & 0xff; while ((v & 0x7f) == 0x7f); }
    uint8_t *dA, *dB; float* dD;
    if (hipMalloc(&dA, A.size()) != hipSuccess || hipMalloc(&dB, B.size()) != hipSuccess ||
        hipMalloc(&dD, (size_t)NT * 256 * 4) != hipSuccess) {
        fprintf(stderr, "hipMalloc failed\n");
        return 1;
    }
    hipMemcpy(dA, A.data(), A.size(), hipMemcpyHostToDevice);
    hipMemcpy(dB, B.data(), B.size(), hipMemcpyHostToDevice);
    hipLaunchKernelGGL(k, dim3(NT), dim3(64), 0, 0, dA, dB, dD, NT);
    std::vector<float> D((size_t)NT * 256);
    hipMemcpy(D.data(), dD, D.size() * 4, hipMemcpyDeviceToHost);
    // two candidate output layouts: lane l, q -> (row 4(l/16)+q, col l%16) or (row l%16, col 4(l/16)+q)
    for (int lay = 0; lay < 2; ++lay) {
        double maxrel = 0, sumrel = 0, maxulp = 0; long n = 0, exact = 0;
        for (int t = 0; t < NT; ++t)
            for (int l = 0; l < 64; ++l)
                for (int q = 0; q < 4; ++q) {
                    int i = lay == 0 ? 4 * (l / 16) + q : l % 16;
                    int j = lay == 0 ? l % 16 : 4 * (l / 16) + q;
                    double ref = 0, mag = 0;
                    for (int kk = 0; kk < 128; ++kk) {
                        double p = e4m3(A[t * 2048 + i * 128 + kk]) * e4m3(B[t * 2048 + j * 128 + kk]);
                        ref += p; mag += std::fabs(p);
                    }
                    double got = D[((size_t)t * 64 + l) * 4 + q];
                    double err = std::fabs(got - ref);
                    double rel = err / mag;   // relative to the sum of magnitudes
                    double ulp = err / std::ldexp(1.0, std::ilogb(std::fabs(ref) > 0 ? std::fabs(ref) : 1e-30) - 23);
                    maxrel = std::max(maxrel, rel); sumrel += rel; ++n;
                    maxulp = std::max(maxulp, ulp);
                    exact += (float)ref == (float)got;
                }
        printf("layout %d: max err/sum|p| = %.3e  mean = %.3e  max ulps of result = %.1f  fp32-rounded-exact %.4f\n",
               lay, maxrel, sumrel / n, maxulp, (double)exact / n);
    }
    return 0;
}
