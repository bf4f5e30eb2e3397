// Host-side launchers of the gfx950 kernels (internal; the public C ABI is
// include/moe.h).  Every launcher only enqueues on `stream` and returns the
// hipError_t of the launch.  Arguments are validated by the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// api.cpp: sets the calling thread's error text (moe_last_error) and returns status
int set_error(int status, const char* fmt, ...);

// route.hip
hipError_t launch_router_logits(const void* x, int x_bf16, int T, int H, const float* wr,
                                const float* bias, int E, float* logits, hipStream_t s);
hipError_t launch_router_topk(const float* logits, int T, int E, int k, int sigmoid,
                              int32_t* ids, float* w, hipStream_t s);

// permute.hip
size_t permute_ws_bytes(int R, int E);
hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* counts, int32_t* offsets,
                          int32_t* src, int32_t* dest, void* ws, hipStream_t s);

// quant.hip
hipError_t launch_quant_e4m3(const void* x, int x_bf16, int rows, int cols, uint8_t* q,
                             float* scale, hipStream_t s);
hipError_t launch_quant_mxfp8(const void* x, int x_bf16, int rows, int cols, uint8_t* q,
                              uint8_t* e8, hipStream_t s);

// combine.hip
// y_mode: 0 fp32, 1 bf16, 2 e4m3 codes + y_scale [rows][H/128]
hipError_t launch_combine(const void* y_perm, int y_mode, const float* y_scale, const void* y_sh, int y_sh_bf16,
                          const int32_t* dest, const float* w, int T, int k, int H, void* out, int out_bf16,
                          hipStream_t s);

// gffn.hip ------------------------------------------------------------------
struct Bank {
    const void* wg; const void* wu; const void* wd;
    const float* sg; const float* su; const float* sd;
    const uint8_t* xgu; const uint8_t* xd;   // MXFP4 exponents in the 16-row tiles' order, or null
};

struct GffnProblem {
    int dt;                       // 0 f32, 1 bf16, 2 e4m3 (activations and weights),
                                  // 3 MXFP4 weights with MXFP8 activations
    const void* a; const float* a_scale; const int32_t* src; int src_div;   // a_scale: E8M0 bytes for MXFP8
    const int32_t* offsets; int G; int R_max;
    Bank routed;
    const void* a_sh; const float* a_sh_scale; int S; int has_shared;
    Bank shared;
    int H, I;
    void* y; void* y_sh; int y_bf16;   // routed outputs bf16 (else fp32 unless y_e4m3)
    int y_e4m3; float* y_scale;        // routed outputs as e4m3 + [R_max][H/128] scales
    int y_sh_bf16;                     // shared outputs bf16 (else fp32)
    // An upper bound on the rows of any group (routed or shared) that the
    // caller guarantees, 0 if none: tile classes no group can reach are then
    // not launched.  The fused layer knows it (T: a token picks an expert at
    // most once); the grouped call alone does not.
    int m_max;
};

size_t gffn_ws_bytes(int R_max, int G, int S, int H, int I, int dt);
// Routed outputs as E4M3 codes (the FP8 combine) are written only by the
// large e4m3 tiles, which need H % 256 == 0 and 32-bit row offsets.
bool gffn_e4m3_y_supported(int H, int I, int R_max, int S);
// MXFP4 exponents into the 16-row streaming tiles' order (see moe_mx_pack_scales).
hipError_t launch_mx_pack_scales(int n, int H, int I, const uint8_t* sg, const uint8_t* su, const uint8_t* sd,
                                 uint8_t* xgu, uint8_t* xd, hipStream_t s);
hipError_t launch_gffn(const GffnProblem& p, void* ws, hipStream_t s);

}  // namespace moe
