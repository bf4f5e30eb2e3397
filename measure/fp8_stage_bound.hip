// What bounds a K stage of the e4m3 large tiles: the stage's direct
// global->LDS loads alone, its MFMA + promotion compute alone, and both
// together, on random e4m3 operands (every finite code but the largest
// magnitudes) and on zero operands.  Persistent grid of one 512-thread
// workgroup per CU, 12 tiles x 56 stages each (a 64-expert gate/up launch:
// 16 weight tiles x 3 m-tiles per expert, n-major with m-tiles innermost, die
// x owning a contiguous chunk); a stage is 256 token rows + 256 weight rows
// of 128 bytes (64 KiB) in a two-buffer LDS ring, 8 waves of 128 x 64
// computed with v_mfma_scale_f32_16x16x128_f8f6f4 and one promotion FMA per
// accumulator and block, as in gffn_big.hip.  "2 in flight" issues the loads
// two stages ahead (into the buffer being computed: a timing variant whose
// numbers are not used).  "half the A reads" reloads a wave's token-row
// fragments only every other 16-row block (timing only, its products are not
// used): the LDS fragment reads of a stage then total 128 KiB instead of 192,
// as four waves of 128 x 128 would read.  Prints per variant the time per
// stage and the shader clock over the run (s_memtime against the 100 MHz
// s_memrealtime).
//
// build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//          measure/fp8_stage_bound.hip -o measure/fp8_stage_bound
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
constexpr int KB = 7168, NST = 56, NE = 64, NT = NE * 16 * 3;
constexpr int kStage = 128, kStageBytes = 65536;
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kStage + ((chunk ^ swz_key(row)) << 4); }
struct Frag8Lane { uint32_t lo, hi; };
__device__ __forceinline__ Frag8Lane frag8_lane(int lane) { const int r = lane % 16, c0 = 2 * (lane / 16); return Frag8Lane{(uint32_t)swz(r, c0), (uint32_t)swz(r, c0 + 1)}; }
__device__ __forceinline__ i32x8 frag8(const uint8_t* base, int row0, const Frag8Lane& fl) {
    const uint8_t* p = base + row0 * kStage;
    const i32x4 lo = *(const i32x4*)(p + fl.lo); const i32x4 hi = *(const i32x4*)(p + fl.hi);
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}
__device__ __forceinline__ void promote1(f32x4& acc, const f32x4& t, float2 c, int j) {
    const float cj = j < 2 ? c.x : c.y;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(t[q], cj, acc[q]);
}
__device__ __forceinline__ void sched_block_order(int nds) {
    if (nds == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) { __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); __builtin_amdgcn_sched_group_barrier(0x002, 4, 0); }
}

__global__ void fill(uint8_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        uint32_t h = (uint32_t)i * 2654435761u; h ^= h >> 15; h *= 2246822519u; h ^= h >> 13;
        uint8_t c = (uint8_t)(h >> 8);
        if ((c & 0x7f) == 0x7f) c = 0x38;
        p[i] = c;
    }
}

template <bool LOADS, bool COMPUTE, int D, bool HALFA = false>
__global__ __launch_bounds__(512) void k(const uint8_t* __restrict__ A, const uint8_t* __restrict__ W, float* out, unsigned long long* clk) {
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wm = wave / 4, wn = wave % 4;
    float* sprod = (float*)(smem + 2 * kStageBytes);
    // LDS starts with operand data (for the variant without loads)
    for (int i = tid; i < 2 * kStageBytes / 16; i += 512) ((i32x4*)smem)[i] = ((const i32x4*)A)[i];
    for (int i = tid; i < 1024; i += 512) sprod[i] = 1.0f + (i & 7) * 1e-3f;
    __syncthreads();
    const int die = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int per_die = NT / 8;
    uint32_t* loffs = (uint32_t*)(smem + 2 * kStageBytes + 4096);   // [8][512], as the production kernel keeps them
    for (int q = 0; q < 8; ++q) loffs[q * 512 + tid] = (uint32_t)((((wave & 3) * 8 + q) * 8 + lane / 8) * KB + (lane % 8) * 16);
    __syncthreads();
    const Frag8Lane fl = frag8_lane(lane);
    float total = 0.f;
    for (int t = die * per_die + slot; t < (die + 1) * per_die; t += 32) {
        const int e = t / 48, n = (t / 3) % 16, m = t % 3;
        const uint8_t* base = wave < 4 ? A + ((size_t)e * 768 + m * 256) * KB : W + ((size_t)e * 4096 + n * 256) * KB;
        auto issue = [&](int s) {
            uint8_t* dst = smem + (s & 1) * kStageBytes + wave * 8192;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                __builtin_amdgcn_global_load_lds((const void*)(base + loffs[q * 512 + tid] + s * 128), (lds_void*)(dst + q * 1024), 16, 0, 0);
        };
        f32x4 acc8[8][4];
        for (int i = 0; i < 8; ++i) for (int j = 0; j < 4; ++j) acc8[i][j] = f32x4{0, 0, 0, 0};
        f32x4 T[4] = {};
        float2 cp = make_float2(0.f, 0.f);
        if (LOADS) { issue(0); if (D == 2) issue(1); }
        for (int s = 0; s < NST; ++s) {
            if (D == 2 && s + 1 < NST) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            const uint8_t* As = smem + (s & 1) * kStageBytes;
            const uint8_t* Bs = As + 256 * kStage;
            if (COMPUTE) {
                const float2* sp2 = (const float2*)(sprod + (s & 1) * 512) + wm * 128 + lane % 16;
                float2 c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = sp2[i * 16];
                i32x8 wfr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int brow = j < 2 ? wn * 32 + 16 * j : 128 + wn * 32 + 16 * (j - 2);
                    wfr[j] = frag8(Bs, brow, fl);
                }
                i32x8 x = frag8(As, wm * 128, fl);
                if (LOADS && s + D < NST) issue(s + D);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    i32x8 xn = x;
                    if (i + 1 < 8 && (!HALFA || (i & 1))) xn = frag8(As, wm * 128 + (i + 1) * 16, fl);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        T[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr[j], x, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
                        if (j == 3) promote1(acc8[i][0], T[0], c[i], 0);
                        else if (i > 0) promote1(acc8[i - 1][j + 1], T[j + 1], c[i - 1], j + 1);
                        else promote1(acc8[7][j + 1], T[j + 1], cp, j + 1);
                    }
                    x = xn;
                    sched_block_order(i + 1 < 8 ? 2 : 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                cp = c[7];
            } else if (LOADS && s + D < NST) {
                issue(s + D);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (int i = 0; i < 8; ++i) for (int j = 0; j < 4; ++j) total += acc8[i][j][0] + acc8[i][j][1] + acc8[i][j][2] + acc8[i][j][3];
        __syncthreads();
    }
    out[blockIdx.x * 512 + tid] = total;
    if (blockIdx.x == 0 && tid == 0) {
        clk[0] = __builtin_amdgcn_s_memtime() - t0;
        clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)
template <bool LOADS, bool COMPUTE, int D = 1, bool HALFA = false>
int run(const char* name, const uint8_t* A, const uint8_t* W, float* out, unsigned long long* clk) {
    auto f = k<LOADS, COMPUTE, D, HALFA>;
    const int lds = 2 * kStageBytes + 4096 + 8 * 512 * 4;
    CK(hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
    float best = 1e9;
    for (int rep = 0; rep < 4; ++rep) {
        CK(hipEventRecord(a));
        hipLaunchKernelGGL(f, dim3(256), dim3(512), lds, 0, A, W, out, clk);
        CK(hipGetLastError());
        CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
        float ms; CK(hipEventElapsedTime(&ms, a, b));
        if (rep > 0 && ms < best) best = ms;
    }
    const double stages = (double)NT / 256 * NST;
    const double flop = (double)NT * NST * 256.0 * 256 * 128 * 2;
    unsigned long long h[2]; CK(hipMemcpy(h, clk, 16, hipMemcpyDeviceToHost));
    printf("%-36s %.3f ms  %.3f us/stage  %.3f PFLOP/s (if computing)  shader clock %.0f MHz\n", name, best, best * 1e3 / stages,
           flop / (best * 1e-3) / 1e15, h[1] ? (double)h[0] / ((double)h[1] / 100.0) : 0.0);
    fflush(stdout);
    return 0;
}

int main() {
    const size_t abytes = (size_t)NE * 768 * KB, wbytes = (size_t)NE * 4096 * KB;
    uint8_t *A, *W; float* out; unsigned long long* clk;
    CK(hipMalloc(&A, abytes)); CK(hipMalloc(&W, wbytes)); CK(hipMalloc(&out, 256 * 512 * 4)); CK(hipMalloc(&clk, 16));
    hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, 0, A, abytes);
    hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, 0, W, wbytes);
    CK(hipDeviceSynchronize());
    int cus = 0; CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    if (cus != 256) { printf("expected 256 CUs, got %d\n", cus); return 1; }
    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            CK(hipMemset(A, 0, abytes)); CK(hipMemset(W, 0, wbytes)); CK(hipDeviceSynchronize());
        }
        printf("--- %s operands\n", pass ? "zero" : "random e4m3");
        if (run<true, false>("loads only", A, W, out, clk)) return 1;
        if (run<true, false, 2>("loads only, 2 in flight", A, W, out, clk)) return 1;
        if (run<false, true>("compute only", A, W, out, clk)) return 1;
        if (run<true, true>("loads + compute", A, W, out, clk)) return 1;
        if (run<true, true, 2>("loads + compute, 2 in flight", A, W, out, clk)) return 1;
        if (run<false, true, 1, true>("compute only, half the A reads", A, W, out, clk)) return 1;
        if (run<true, true, 1, true>("loads + compute, half the A reads", A, W, out, clk)) return 1;
    }
    return 0;
}
