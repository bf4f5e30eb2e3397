// moe_probe: a native driver of the C ABI (no Python, no torch), used for
// hardware-counter runs (rocprofv3 --pmc) and quick timing.
//
//   moe_probe decode  [iters]   T=128,   H=7168, 256+1 experts, I=2048, top-8, bf16, fp32 out
//   moe_probe skew    [iters]   T=4096,  same layer, additive logit bias on 20 experts
//   moe_probe prefill [iters]   T=16384, same layer with e4m3 block-scaled weights, bf16 out
//   moe_probe decode-mxfp4 [iters]  the decode layer with MXFP4 expert weights
//   moe_probe copy    [iters]   a plain device copy of 1 GiB (counter calibration)
//   moe_probe file DIR [iters]  the workload described by DIR/meta.txt (written by
//                               bench.py --dump-inputs): a layer with the dumped
//                               tokens, router and bias (so its routing is the
//                               benchmark's), or the pre-routed grouped FFN with
//                               the dumped group sizes
//
// Inputs are filled on the device from a hash of the element index (uniform
// values with the layer's scales); values matter here only through the
// routing distribution, which is close to uniform except for `skew`.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <fstream>
#include <map>
#include <sstream>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "moe.h"

#define CK(x)                                                                         \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

#define CM(x)                                                                         \
    do {                                                                              \
        moe_status_t s_ = (x);                                                        \
        if (s_ != MOE_OK) {                                                           \
            fprintf(stderr, "%s: %s (%s)\n", #x, moe_status_string(s_), moe_last_error()); \
            exit(3);                                                                  \
        }                                                                             \
    } while (0)

__device__ __forceinline__ uint32_t hash32(uint64_t x) {
    x ^= x >> 33;
    x *= 0xff51afd7ed558ccdull;
    x ^= x >> 33;
    x *= 0xc4ceb9fe1a85ec53ull;
    x ^= x >> 33;
    return (uint32_t)x;
}

// uniform in [-a, a)
__device__ __forceinline__ float uni(uint64_t seed, size_t i, float a) {
    return ((float)hash32(seed * 0x9E3779B97F4A7C15ull + i) * (1.0f / 2147483648.0f) - 1.0f) * a;
}

__global__ void fill_f32(float* p, size_t n, uint64_t seed, float a) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = uni(seed, i, a);
}

__global__ void fill_bf16(uint16_t* p, size_t n, uint64_t seed, float a) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const uint32_t u = __float_as_uint(uni(seed, i, a));
        p[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
}

// random finite e4m3 codes with magnitude exponent <= 2^3 (no NaN)
__global__ void fill_e4m3(uint8_t* p, size_t n, uint64_t seed) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const uint32_t h = hash32(seed * 0x9E3779B97F4A7C15ull + i);
        p[i] = (uint8_t)((h & 0x80u) | (h % 0x50u));
    }
}

// bytes lo + (hash % span): E2M1 code pairs (0, 256) or E8M0 exponents
__global__ void fill_u8(uint8_t* p, size_t n, uint64_t seed, uint32_t lo, uint32_t span) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = (uint8_t)(lo + hash32(seed * 0x9E3779B97F4A7C15ull + i) % span);
}

__global__ void copy_u4(const uint4* __restrict__ s, uint4* __restrict__ d, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        d[i] = s[i];
}

static void* dalloc(size_t bytes) {
    void* p = nullptr;
    CK(hipMalloc(&p, bytes < 256 ? 256 : bytes));
    return p;
}

struct BankBuf {
    moe_experts_t d;
};

static BankBuf make_bank(int n, int H, int I, int dt, uint64_t seed) {
    BankBuf b{};
    const size_t ne = (size_t)n * H * I;
    const size_t eb = dt == MOE_E4M3 ? 1 : dt == MOE_BF16 ? 2 : 4;
    const size_t nb = dt == MOE_MXFP4 ? ne / 2 : ne * eb;
    void* g = dalloc(nb);
    void* u = dalloc(nb);
    void* w = dalloc(nb);
    if (dt == MOE_MXFP4) {
        // uniform E2M1 codes, exponents 2^-8 / 2^-7 (weights of rms about 0.018)
        uint8_t* e[3];
        for (int j = 0; j < 3; ++j) {
            hipLaunchKernelGGL(fill_u8, dim3(4096), dim3(256), 0, 0, (uint8_t*)(j == 0 ? g : j == 1 ? u : w), nb,
                               seed + 1 + j, 0u, 256u);
            e[j] = (uint8_t*)dalloc(ne / 32);
            hipLaunchKernelGGL(fill_u8, dim3(4096), dim3(256), 0, 0, e[j], ne / 32, seed + 11 + j, 119u, 2u);
        }
        b.d.s_gate = e[0]; b.d.s_up = e[1]; b.d.s_down = e[2];
    } else if (dt == MOE_E4M3) {
        hipLaunchKernelGGL(fill_e4m3, dim3(4096), dim3(256), 0, 0, (uint8_t*)g, ne, seed + 1);
        hipLaunchKernelGGL(fill_e4m3, dim3(4096), dim3(256), 0, 0, (uint8_t*)u, ne, seed + 2);
        hipLaunchKernelGGL(fill_e4m3, dim3(4096), dim3(256), 0, 0, (uint8_t*)w, ne, seed + 3);
        const size_t ns = (size_t)n * (H / 128) * (I / 128);
        float* sg = (float*)dalloc(ns * 4);
        float* su = (float*)dalloc(ns * 4);
        float* sd = (float*)dalloc(ns * 4);
        for (float* s : {sg, su, sd}) hipLaunchKernelGGL(fill_f32, dim3(256), dim3(256), 0, 0, s, ns, seed + 7, 1e-3f);
        b.d.s_gate = sg; b.d.s_up = su; b.d.s_down = sd;
    } else if (dt == MOE_F32) {
        const float a = 0.0346f;
        hipLaunchKernelGGL(fill_f32, dim3(4096), dim3(256), 0, 0, (float*)g, ne, seed + 1, a);
        hipLaunchKernelGGL(fill_f32, dim3(4096), dim3(256), 0, 0, (float*)u, ne, seed + 2, a);
        hipLaunchKernelGGL(fill_f32, dim3(4096), dim3(256), 0, 0, (float*)w, ne, seed + 3, a);
    } else {
        const float a = 0.0346f;   // uniform with standard deviation 0.02
        hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, (uint16_t*)g, ne, seed + 1, a);
        hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, (uint16_t*)u, ne, seed + 2, a);
        hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, (uint16_t*)w, ne, seed + 3, a);
    }
    b.d.n = n; b.d.H = H; b.d.I = I; b.d.dt = dt;
    b.d.w_gate = g; b.d.w_up = u; b.d.w_down = w;
    if (dt == MOE_MXFP4 && H % 1024 == 0 && I % 512 == 0) {
        // the exponents packed for the 16-row tiles, as the Python banks carry them
        void* xgu = dalloc(2 * ne / 32);
        void* xd = dalloc(ne / 32);
        if (moe_mx_pack_scales(&b.d, xgu, xd, nullptr) != MOE_OK) {
            std::fprintf(stderr, "moe_mx_pack_scales: %s\n", moe_last_error());
            std::exit(1);
        }
        b.d.s_gate_up_packed = xgu; b.d.s_down_packed = xd;
    }
    return b;
}

static std::map<std::string, std::string> read_meta(const std::string& dir) {
    std::map<std::string, std::string> m;
    std::ifstream f(dir + "/meta.txt");
    if (!f) {
        fprintf(stderr, "cannot read %s/meta.txt\n", dir.c_str());
        exit(1);
    }
    std::string line;
    while (std::getline(f, line)) {
        const size_t sp = line.find(' ');
        if (sp != std::string::npos) m[line.substr(0, sp)] = line.substr(sp + 1);
    }
    return m;
}

static void* load_file(const std::string& path, size_t bytes) {
    std::vector<char> h(bytes);
    FILE* f = fopen(path.c_str(), "rb");
    if (!f || fread(h.data(), 1, bytes, f) != bytes) {
        fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path.c_str());
        exit(1);
    }
    fclose(f);
    void* d = dalloc(bytes);
    CK(hipMemcpy(d, h.data(), bytes, hipMemcpyHostToDevice));
    return d;
}

static int dt_of(const std::string& s) {
    return s == "f32" ? MOE_F32 : s == "bf16" ? MOE_BF16 : s == "mxfp4" ? MOE_MXFP4 : MOE_E4M3;
}

int main(int argc, char** argv) {
    const std::string mode = argc > 1 ? argv[1] : "decode";
    const std::string dir = (mode == "file" && argc > 2) ? argv[2] : "";
    const int iters = mode == "file" ? (argc > 3 ? atoi(argv[3]) : 5) : (argc > 2 ? atoi(argv[2]) : 5);
    hipStream_t st;
    CK(hipStreamCreate(&st));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));

    if (mode == "copy") {
        const size_t bytes = (size_t)1 << 30;
        void* s = dalloc(bytes);
        void* d = dalloc(bytes);
        CK(hipMemsetAsync(s, 1, bytes, st));
        const size_t n = bytes / 16;
        hipLaunchKernelGGL(copy_u4, dim3(8192), dim3(256), 0, st, (const uint4*)s, (uint4*)d, n);
        CK(hipEventRecord(e0, st));
        for (int i = 0; i < iters; ++i)
            hipLaunchKernelGGL(copy_u4, dim3(8192), dim3(256), 0, st, (const uint4*)s, (uint4*)d, n);
        CK(hipEventRecord(e1, st));
        CK(hipEventSynchronize(e1));
        float ms = 0;
        CK(hipEventElapsedTime(&ms, e0, e1));
        printf("copy 1 GiB: %.3f ms/iter, %.1f GB/s (read+write)\n", ms / iters, 2.0 * bytes / (ms / iters * 1e-3) / 1e9);
        return 0;
    }

    if (mode == "file") {
        auto m = read_meta(dir);
        if (m["kind"] == "grouped") {
            const int H = std::stoi(m["H"]), I = std::stoi(m["I"]), S = std::stoi(m["shared_rows"]);
            const int dt = dt_of(m["dt"]);
            std::vector<int> offs{0};
            std::istringstream gs(m["groups"]);
            for (int g; gs >> g;) offs.push_back(offs.back() + g);
            const int G = (int)offs.size() - 1, R = offs.back();
            const bool q8 = dt == MOE_E4M3 || dt == MOE_MXFP4;
            const size_t eb = q8 ? 1 : dt == MOE_BF16 ? 2 : 4;
            void* a = dalloc((size_t)(R + S) * H * eb);
            float* as = (float*)dalloc((size_t)(R + S) * (H / 128) * 4);   // also holds [R+S][H/32] E8M0 bytes
            if (q8) hipLaunchKernelGGL(fill_e4m3, dim3(4096), dim3(256), 0, 0, (uint8_t*)a, (size_t)(R + S) * H, 21);
            else hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, (uint16_t*)a, (size_t)(R + S) * H, 21, 1.73f);
            if (dt == MOE_MXFP4)
                hipLaunchKernelGGL(fill_u8, dim3(256), dim3(256), 0, 0, (uint8_t*)as, (size_t)(R + S) * (H / 32), 22, 118u, 4u);
            else
                hipLaunchKernelGGL(fill_f32, dim3(256), dim3(256), 0, 0, as, (size_t)(R + S) * (H / 128), 22, 1e-2f);
            int32_t* d_offs = (int32_t*)dalloc(offs.size() * 4);
            CK(hipMemcpy(d_offs, offs.data(), offs.size() * 4, hipMemcpyHostToDevice));
            BankBuf routed = make_bank(G, H, I, dt, 100);
            BankBuf shared = make_bank(1, H, I, dt, 200);
            void* y = dalloc((size_t)R * H * 2);
            void* y_sh = dalloc((size_t)(S > 0 ? S : 1) * H * 2);
            const size_t wsb = moe_grouped_ffn_workspace_size(R, G, S, H, I, dt);
            void* ws = dalloc(wsb);
            CK(hipDeviceSynchronize());
            auto run = [&]() {
                const void* ash = !q8 || S == 0 ? nullptr
                                : dt == MOE_MXFP4 ? (const void*)((const uint8_t*)as + (size_t)R * (H / 32))
                                                  : (const void*)(as + (size_t)R * (H / 128));
                CM(moe_grouped_ffn(a, dt == MOE_MXFP4 ? MOE_MXFP8 : dt, q8 ? as : nullptr, nullptr, 1, d_offs, G, R, &routed.d,
                                   S > 0 ? (const uint8_t*)a + (size_t)R * H * eb : nullptr, ash, S,
                                   S > 0 ? &shared.d : nullptr, y, MOE_BF16, nullptr, S > 0 ? y_sh : nullptr, MOE_BF16,
                                   ws, wsb, st));
            };
            run();
            CK(hipEventRecord(e0, st));
            for (int i = 0; i < iters; ++i) run();
            CK(hipEventRecord(e1, st));
            CK(hipEventSynchronize(e1));
            float ms = 0;
            CK(hipEventElapsedTime(&ms, e0, e1));
            printf("file %s: grouped G=%d R=%d S=%d %.3f ms/call\n", dir.c_str(), G, R, S, ms / iters);
            return 0;
        }
    }

    int T, x_dt = MOE_BF16, w_dt, out_dt;
    bool bias = false;
    if (mode == "decode") { T = 128; w_dt = MOE_BF16; out_dt = MOE_F32; }
    else if (mode == "skew") { T = 4096; w_dt = MOE_BF16; out_dt = MOE_F32; bias = true; }
    else if (mode == "prefill") { T = 16384; w_dt = MOE_E4M3; out_dt = MOE_BF16; }
    else if (mode == "decode-mxfp4") { T = 128; w_dt = MOE_MXFP4; out_dt = MOE_F32; }
    else if (mode != "file") { fprintf(stderr, "unknown mode %s\n", mode.c_str()); return 1; }
    int H = 7168, E = 256, k = 8, I = 2048, score = MOE_SIGMOID, has_shared = 1, y_dt = -1;
    void* x = nullptr;
    float* wr = nullptr;
    float* b = nullptr;
    if (mode == "file") {
        auto m = read_meta(dir);
        T = std::stoi(m["T"]); H = std::stoi(m["H"]); E = std::stoi(m["E"]); k = std::stoi(m["k"]); I = std::stoi(m["I"]);
        x_dt = dt_of(m["x_dt"]); w_dt = dt_of(m["w_dt"]); out_dt = dt_of(m["out_dt"]);
        score = m["score"] == "softmax" ? MOE_SOFTMAX : MOE_SIGMOID;
        has_shared = std::stoi(m["shared"]);
        if (m.count("y_dt")) y_dt = dt_of(m["y_dt"]);
        x = load_file(dir + "/x.bin", (size_t)T * H * (x_dt == MOE_F32 ? 4 : 2));
        wr = (float*)load_file(dir + "/w_router.bin", (size_t)H * E * 4);
        if (std::stoi(m["bias"])) b = (float*)load_file(dir + "/bias.bin", (size_t)E * 4);
    } else {
        x = dalloc((size_t)T * H * 2);
        hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, (uint16_t*)x, (size_t)T * H, 11, 1.73f);
        wr = (float*)dalloc((size_t)H * E * 4);
        hipLaunchKernelGGL(fill_f32, dim3(4096), dim3(256), 0, 0, wr, (size_t)H * E, 12, 1.73f / 84.7f);
        if (bias) {
            std::vector<float> hb(E, -1.0f);
            for (int e = 0; e < 20; ++e) hb[(e * 37) % E] = 2.5f;   // 20 hot experts
            b = (float*)dalloc(E * 4);
            CK(hipMemcpy(b, hb.data(), E * 4, hipMemcpyHostToDevice));
        }
    }
    BankBuf routed = make_bank(E, H, I, w_dt, 100);
    BankBuf shared = make_bank(1, H, I, w_dt, 200);
    void* out = dalloc((size_t)T * H * (out_dt == MOE_BF16 ? 2 : 4));
    if (y_dt < 0) y_dt = out_dt;
    const size_t wsb = moe_layer_workspace_size(T, H, E, k, I, x_dt, w_dt, has_shared, out_dt, y_dt);
    void* ws = dalloc(wsb);
    CK(hipDeviceSynchronize());

    auto run = [&]() {
        CM(moe_layer(x, x_dt, T, H, wr, b, E, k, score, &routed.d, has_shared ? &shared.d : nullptr, out, out_dt, y_dt, nullptr,
                     nullptr, nullptr, ws, wsb, st));
    };
    run();
    CK(hipEventRecord(e0, st));
    for (int i = 0; i < iters; ++i) run();
    CK(hipEventRecord(e1, st));
    CK(hipEventSynchronize(e1));
    float ms = 0;
    CK(hipEventElapsedTime(&ms, e0, e1));
    printf("%s: T=%d %.3f ms/layer, %.0f tokens/s\n", mode.c_str(), T, ms / iters, T / (ms / iters * 1e-3));
    return 0;
}
