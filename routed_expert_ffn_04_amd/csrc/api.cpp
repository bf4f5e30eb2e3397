// C ABI of the sparse MoE FFN layer (declarations and contracts: include/moe.h).
// Validation, workspace carving and kernel launches; no allocation, no
// host synchronisation.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status_t hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    g_err[0] = 0;
    return MOE_OK;
}

size_t al(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status_t check_bank(const moe_experts_t* b, int n, int H, int I, const char* name) {
    if (!b) return fail(MOE_ERR_INVALID, "%s: null bank", name);
    if (b->n != n) return fail(MOE_ERR_INVALID, "%s: n = %d, expected %d", name, b->n, n);
    if (b->H != H || b->I != I) return fail(MOE_ERR_INVALID, "%s: H/I = %d/%d, expected %d/%d", name, b->H, b->I, H, I);
    if (b->dt != MOE_F32 && b->dt != MOE_BF16 && b->dt != MOE_E4M3 && b->dt != MOE_MXFP4)
        return fail(MOE_ERR_UNSUPPORTED, "%s: weight dtype %d", name, b->dt);
    if (!b->w_gate || !b->w_up || !b->w_down) return fail(MOE_ERR_INVALID, "%s: null weight pointer", name);
    if (!aligned16(b->w_gate) || !aligned16(b->w_up) || !aligned16(b->w_down))
        return fail(MOE_ERR_INVALID, "%s: weights must be 16-byte aligned", name);
    if ((b->dt == MOE_E4M3 || b->dt == MOE_MXFP4) && (!b->s_gate || !b->s_up || !b->s_down))
        return fail(MOE_ERR_INVALID, "%s: E4M3 / MXFP4 bank without scales", name);
    if (b->dt == MOE_MXFP4 && (((uintptr_t)b->s_gate | (uintptr_t)b->s_up | (uintptr_t)b->s_down) & 3u))
        return fail(MOE_ERR_INVALID, "%s: MXFP4 exponents must be 4-byte aligned", name);
    if ((b->s_gate_up_packed || b->s_down_packed) &&
        (b->dt != MOE_MXFP4 || H % 1024 != 0 || I % 512 != 0))
        return fail(MOE_ERR_UNSUPPORTED, "%s: packed exponents need MXFP4 weights, H %% 1024 == 0 and I %% 512 == 0",
                    name);
    if (!aligned16(b->s_gate_up_packed) || !aligned16(b->s_down_packed))
        return fail(MOE_ERR_INVALID, "%s: packed exponents must be 16-byte aligned", name);
    return MOE_OK;
}

moe::Bank to_bank(const moe_experts_t* b) {
    moe::Bank k{};
    if (!b) return k;
    k.wg = b->w_gate; k.wu = b->w_up; k.wd = b->w_down;
    // fp32 block scales (E4M3) or E8M0 exponent bytes (MXFP4), by the bank's dtype
    k.sg = (const float*)b->s_gate; k.su = (const float*)b->s_up; k.sd = (const float*)b->s_down;
    k.xgu = (const uint8_t*)b->s_gate_up_packed; k.xd = (const uint8_t*)b->s_down_packed;
    return k;
}

}  // namespace

namespace moe {
int set_error(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}
}  // namespace moe

extern "C" {

const char* moe_status_string(int32_t st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error(void) { return g_err; }

// ------------------------------------------------------------------ route
size_t moe_route_workspace_size(int32_t T, int32_t E) {
    if (T < 0 || E < 0) return 0;
    return al((size_t)T * E * sizeof(float));
}

static moe_status_t validate_route(const void* x, int32_t x_dt, int32_t T, int32_t H, const float* wr,
                                   int32_t E, int32_t k, int32_t score) {
    if (T < 0 || H <= 0 || E <= 0 || k <= 0) return fail(MOE_ERR_INVALID, "route: T=%d H=%d E=%d k=%d", T, H, E, k);
    if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "route: E=%d > 1024", E);
    if (k > E) return fail(MOE_ERR_INVALID, "route: k=%d > E=%d", k, E);
    if (H % 128) return fail(MOE_ERR_UNSUPPORTED, "route: H=%d not a multiple of 128", H);
    if (x_dt != MOE_F32 && x_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "route: x dtype %d", x_dt);
    if (score != MOE_SOFTMAX && score != MOE_SIGMOID) return fail(MOE_ERR_INVALID, "route: score %d", score);
    if (T > 0 && (!x || !wr)) return fail(MOE_ERR_INVALID, "route: null x or w_router");
    return MOE_OK;
}

moe_status_t moe_route(const void* x, int32_t x_dt, int32_t T, int32_t H, const float* w_router,
                       const float* bias, int32_t E, int32_t k, int32_t score, int32_t* topk_ids,
                       float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    moe_status_t st = validate_route(x, x_dt, T, H, w_router, E, k, score);
    if (st) return st;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !topk_w) return fail(MOE_ERR_INVALID, "route: null output");
    if (!ws || ws_bytes < moe_route_workspace_size(T, E)) return fail(MOE_ERR_WORKSPACE, "route: workspace");
    hipStream_t s = (hipStream_t)stream;
    float* logits = (float*)ws;
    hipError_t e = moe::launch_router_logits(x, x_dt == MOE_BF16, T, H, w_router, bias, E, logits, s);
    if (e == hipSuccess) e = moe::launch_router_topk(logits, T, E, k, score == MOE_SIGMOID, topk_ids, topk_w, s);
    return hip_check(e, "moe_route");
}

// ------------------------------------------------------------------ permute
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
    if (T < 0 || k <= 0 || E <= 0 || (long long)T * k > (1LL << 30)) return 0;
    return al(moe::permute_ws_bytes(T * k, E));
}

moe_status_t moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                         int32_t* offsets, int32_t* src, int32_t* dest, void* ws, size_t ws_bytes,
                         void* stream) {
    if (T < 0 || k <= 0 || E <= 0) return fail(MOE_ERR_INVALID, "permute: T=%d k=%d E=%d", T, k, E);
    if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "permute: E=%d > 1024", E);
    if ((long long)T * k > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "permute: T*k too large");
    if (!counts || !offsets) return fail(MOE_ERR_INVALID, "permute: null counts/offsets");
    if (T > 0 && (!topk_ids || !src || !dest)) return fail(MOE_ERR_INVALID, "permute: null pointer");
    if (!ws || ws_bytes < moe_permute_workspace_size(T, k, E)) return fail(MOE_ERR_WORKSPACE, "permute: workspace");
    return hip_check(moe::launch_permute(topk_ids, T * k, E, counts, offsets, src, dest, ws, (hipStream_t)stream),
                     "moe_permute");
}

// ------------------------------------------------------------------ quant
moe_status_t moe_quant_e4m3_1x128(const void* x, int32_t x_dt, int32_t rows, int32_t cols, uint8_t* q,
                                  float* scale, void* stream) {
    if (rows < 0 || cols <= 0) return fail(MOE_ERR_INVALID, "quant: rows=%d cols=%d", rows, cols);
    if (cols % 128) return fail(MOE_ERR_UNSUPPORTED, "quant: cols=%d not a multiple of 128", cols);
    if (x_dt != MOE_F32 && x_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "quant: x dtype %d", x_dt);
    if (rows == 0) return MOE_OK;
    if (!x || !q || !scale) return fail(MOE_ERR_INVALID, "quant: null pointer");
    if (!aligned16(x) || ((uintptr_t)q & 7u)) return fail(MOE_ERR_INVALID, "quant: misaligned x or q");
    return hip_check(moe::launch_quant_e4m3(x, x_dt == MOE_BF16, rows, cols, q, scale, (hipStream_t)stream),
                     "moe_quant_e4m3_1x128");
}

moe_status_t moe_quant_mxfp8(const void* x, int32_t x_dt, int32_t rows, int32_t cols, uint8_t* q, uint8_t* e8m0,
                             void* stream) {
    if (rows < 0 || cols <= 0) return fail(MOE_ERR_INVALID, "quant_mxfp8: rows=%d cols=%d", rows, cols);
    if (cols % 32) return fail(MOE_ERR_UNSUPPORTED, "quant_mxfp8: cols=%d not a multiple of 32", cols);
    if (x_dt != MOE_F32 && x_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "quant_mxfp8: x dtype %d", x_dt);
    if (rows == 0) return MOE_OK;
    if (!x || !q || !e8m0) return fail(MOE_ERR_INVALID, "quant_mxfp8: null pointer");
    if (!aligned16(x) || ((uintptr_t)q & 7u)) return fail(MOE_ERR_INVALID, "quant_mxfp8: misaligned x or q");
    return hip_check(moe::launch_quant_mxfp8(x, x_dt == MOE_BF16, rows, cols, q, e8m0, (hipStream_t)stream),
                     "moe_quant_mxfp8");
}

// ------------------------------------------------------------------ grouped FFN
size_t moe_grouped_ffn_workspace_size(int32_t R_max, int32_t G, int32_t S, int32_t H, int32_t I, int32_t w_dt) {
    if (R_max < 0 || G < 0 || S < 0 || H <= 0 || I <= 0) return 0;
    return al(moe::gffn_ws_bytes(R_max, G, S, H, I, w_dt));
}

moe_status_t moe_grouped_ffn(const void* a, int32_t a_dt, const void* a_scale, const int32_t* src,
                             int32_t src_div, const int32_t* offsets, int32_t G, int32_t R_max,
                             const moe_experts_t* routed, const void* a_sh, const void* a_sh_scale,
                             int32_t S, const moe_experts_t* shared, void* y, int32_t y_dt, float* y_scale,
                             void* y_sh, int32_t y_sh_dt, void* ws, size_t ws_bytes, void* stream) {
    if (G < 0 || R_max < 0 || S < 0) return fail(MOE_ERR_INVALID, "grouped_ffn: G=%d R_max=%d S=%d", G, R_max, S);
    if (G > 1024) return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: G=%d > 1024", G);
    if (G > 0 && !routed) return fail(MOE_ERR_INVALID, "grouped_ffn: null routed bank");
    const moe_experts_t* ref = routed ? routed : shared;
    if (!ref) return fail(MOE_ERR_INVALID, "grouped_ffn: no bank");
    const int H = ref->H, I = ref->I;
    if (H <= 0 || I <= 0 || H % 128 || I % 128)
        return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: H=%d I=%d must be positive multiples of 128", H, I);
    moe_status_t st;
    if (routed && (st = check_bank(routed, G, H, I, "routed"))) return st;
    if (shared && (st = check_bank(shared, 1, H, I, "shared"))) return st;
    const int wdt = ref->dt;
    if (shared && shared->dt != wdt) return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: shared/routed dtype differ");
    const int want_adt = wdt == MOE_MXFP4 ? MOE_MXFP8 : wdt;
    if (a_dt != want_adt)
        return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: activation dtype %d with weights %d", a_dt, wdt);
    if (y_dt != MOE_F32 && y_dt != MOE_BF16 && y_dt != MOE_E4M3)
        return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: y dtype %d", y_dt);
    if (y_dt == MOE_E4M3 &&
        (wdt != MOE_E4M3 || !moe::gffn_e4m3_y_supported(H, I, R_max, shared && S > 0 ? S : 0)))
        return fail(MOE_ERR_UNSUPPORTED,
                    "grouped_ffn: E4M3 y needs E4M3 weights, H %% 256 == 0 and row offsets within 32 bits "
                    "(H=%d I=%d R_max=%d S=%d)", H, I, R_max, S);
    if (y_sh_dt != MOE_F32 && y_sh_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: y_sh dtype %d", y_sh_dt);
    if (src && src_div <= 0) return fail(MOE_ERR_INVALID, "grouped_ffn: src_div=%d", src_div);
    const bool has_sh = shared && S > 0;
    if (R_max > 0 && G > 0 && (!a || !offsets || !y)) return fail(MOE_ERR_INVALID, "grouped_ffn: null a/offsets/y");
    if (R_max > 0 && G > 0 && y_dt == MOE_E4M3 && !y_scale) return fail(MOE_ERR_INVALID, "grouped_ffn: E4M3 y without y_scale");
    if (has_sh && (!a_sh || !y_sh)) return fail(MOE_ERR_INVALID, "grouped_ffn: null a_sh/y_sh");
    if ((wdt == MOE_E4M3 || wdt == MOE_MXFP4) && ((R_max > 0 && G > 0 && !a_scale) || (has_sh && !a_sh_scale)))
        return fail(MOE_ERR_INVALID, "grouped_ffn: E4M3 / MXFP8 activations without scales");
    if (wdt == MOE_MXFP4 && (((uintptr_t)a_scale | (uintptr_t)a_sh_scale) & 3u))
        return fail(MOE_ERR_INVALID, "grouped_ffn: MXFP8 exponents must be 4-byte aligned");
    if ((a && !aligned16(a)) || (a_sh && !aligned16(a_sh))) return fail(MOE_ERR_INVALID, "grouped_ffn: misaligned a");
    if ((R_max == 0 || G == 0) && !has_sh) return MOE_OK;
    if (G == 0) return fail(MOE_ERR_UNSUPPORTED, "grouped_ffn: the shared expert alone (G = 0) is not supported");
    if (!offsets) return fail(MOE_ERR_INVALID, "grouped_ffn: null offsets");
    if (!ws || ws_bytes < moe_grouped_ffn_workspace_size(R_max, G, has_sh ? S : 0, H, I, wdt))
        return fail(MOE_ERR_WORKSPACE, "grouped_ffn: workspace");
    moe::GffnProblem p{};
    p.dt = wdt; p.a = a; p.a_scale = (const float*)a_scale; p.src = src; p.src_div = src ? src_div : 1;
    p.offsets = offsets; p.G = G; p.R_max = R_max;
    p.routed = to_bank(routed);
    p.a_sh = a_sh; p.a_sh_scale = (const float*)a_sh_scale; p.S = has_sh ? S : 0; p.has_shared = has_sh;
    p.shared = to_bank(shared);
    p.H = H; p.I = I; p.y = y; p.y_sh = y_sh; p.y_bf16 = (y_dt == MOE_BF16);
    p.y_e4m3 = (y_dt == MOE_E4M3); p.y_scale = y_scale; p.y_sh_bf16 = (y_sh_dt == MOE_BF16);
    return hip_check(moe::launch_gffn(p, ws, (hipStream_t)stream), "moe_grouped_ffn");
}

// ------------------------------------------------------------------ packed MXFP4 exponents
moe_status_t moe_mx_pack_scales(const moe_experts_t* bank, void* s_gate_up_packed, void* s_down_packed,
                                void* stream) {
    if (!bank) return fail(MOE_ERR_INVALID, "mx_pack_scales: null bank");
    if (bank->dt != MOE_MXFP4) return fail(MOE_ERR_UNSUPPORTED, "mx_pack_scales: weight dtype %d", bank->dt);
    const int n = bank->n, H = bank->H, I = bank->I;
    if (n < 0 || H <= 0 || I <= 0) return fail(MOE_ERR_INVALID, "mx_pack_scales: n=%d H=%d I=%d", n, H, I);
    if (H % 1024 != 0 || I % 512 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "mx_pack_scales: needs H %% 1024 == 0 and I %% 512 == 0 (H=%d I=%d)", H, I);
    if (s_gate_up_packed && (!bank->s_gate || !bank->s_up))
        return fail(MOE_ERR_INVALID, "mx_pack_scales: null s_gate / s_up");
    if (s_down_packed && !bank->s_down) return fail(MOE_ERR_INVALID, "mx_pack_scales: null s_down");
    if (!aligned16(s_gate_up_packed) || !aligned16(s_down_packed))
        return fail(MOE_ERR_INVALID, "mx_pack_scales: outputs must be 16-byte aligned");
    if (n == 0 || (!s_gate_up_packed && !s_down_packed)) return MOE_OK;
    return hip_check(moe::launch_mx_pack_scales(n, H, I, (const uint8_t*)bank->s_gate, (const uint8_t*)bank->s_up,
                                                (const uint8_t*)bank->s_down, (uint8_t*)s_gate_up_packed,
                                                (uint8_t*)s_down_packed, (hipStream_t)stream),
                     "moe_mx_pack_scales");
}

// ------------------------------------------------------------------ combine
moe_status_t moe_combine(const void* y_perm, int32_t y_dt, const float* y_scale, const void* y_sh,
                         int32_t y_sh_dt, const int32_t* dest, const float* topk_w, int32_t T, int32_t k,
                         int32_t H, void* out, int32_t out_dt, void* stream) {
    if (T < 0 || k <= 0 || H <= 0) return fail(MOE_ERR_INVALID, "combine: T=%d k=%d H=%d", T, k, H);
    if (H % 128) return fail(MOE_ERR_UNSUPPORTED, "combine: H=%d not a multiple of 128", H);
    if (y_dt != MOE_F32 && y_dt != MOE_BF16 && y_dt != MOE_E4M3)
        return fail(MOE_ERR_UNSUPPORTED, "combine: y dtype %d", y_dt);
    if (y_sh && y_sh_dt != MOE_F32 && y_sh_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "combine: y_sh dtype %d", y_sh_dt);
    if (out_dt != MOE_F32 && out_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "combine: out dtype %d", out_dt);
    if (T == 0) return MOE_OK;
    if (!y_perm || !dest || !topk_w || !out) return fail(MOE_ERR_INVALID, "combine: null pointer");
    if (y_dt == MOE_E4M3 && !y_scale) return fail(MOE_ERR_INVALID, "combine: E4M3 y without y_scale");
    if (!aligned16(y_perm) || (y_sh && !aligned16(y_sh)) || !aligned16(out))
        return fail(MOE_ERR_INVALID, "combine: misaligned y or out");
    const int ym = y_dt == MOE_E4M3 ? 2 : y_dt == MOE_BF16 ? 1 : 0;
    return hip_check(moe::launch_combine(y_perm, ym, y_scale, y_sh, y_sh_dt == MOE_BF16, dest, topk_w, T, k, H, out,
                                         out_dt == MOE_BF16, (hipStream_t)stream),
                     "moe_combine");
}

// ------------------------------------------------------------------ layer
namespace {
struct LayerWs {
    size_t logits, ids, w, counts, offsets, src, dest, perm, xq, xs, yperm, yscale, ysh, gffn, total;
};

LayerWs layer_ws(int T, int H, int E, int k, int I, int x_dt, int w_dt, int has_sh, int out_dt, int y_dt) {
    (void)x_dt;
    LayerWs L{};
    const size_t R = (size_t)T * k;
    const size_t yb = out_dt == MOE_BF16 ? 2 : 4;                                   // y_sh
    const size_t ypb = y_dt == MOE_E4M3 ? 1 : y_dt == MOE_BF16 ? 2 : 4;             // y_perm
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t r = o; o += al(bytes); return r; };
    L.logits = take((size_t)T * E * 4);
    L.ids = take(R * 4);
    L.w = take(R * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.src = take(R * 4);
    L.dest = take(R * 4);
    L.perm = take(moe::permute_ws_bytes((int)R, E));
    const bool q8 = w_dt == MOE_E4M3 || w_dt == MOE_MXFP4;               // x quantised in-layer
    L.xq = take(q8 ? (size_t)T * H : 0);
    L.xs = take(q8 ? (w_dt == MOE_E4M3 ? (size_t)T * (H / 128) * 4 : (size_t)T * (H / 32)) : 0);
    L.yperm = take(R * H * ypb);
    L.yscale = take(y_dt == MOE_E4M3 ? R * (H / 128) * 4 : 0);
    L.ysh = take(has_sh ? (size_t)T * H * yb : 0);
    L.gffn = take(moe::gffn_ws_bytes((int)R, E, has_sh ? T : 0, H, I, w_dt));
    L.total = o;
    return L;
}
}  // namespace

size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t E, int32_t k, int32_t I, int32_t x_dt,
                                int32_t w_dt, int32_t has_shared, int32_t out_dt, int32_t y_dt) {
    if (T < 0 || H <= 0 || E <= 0 || k <= 0 || I <= 0) return 0;
    return layer_ws(T, H, E, k, I, x_dt, w_dt, has_shared, out_dt, y_dt).total;
}

moe_status_t moe_layer(const void* x, int32_t x_dt, int32_t T, int32_t H, const float* w_router,
                       const float* bias, int32_t E, int32_t k, int32_t score, const moe_experts_t* routed,
                       const moe_experts_t* shared, void* out, int32_t out_dt, int32_t y_dt, int32_t* topk_ids_out,
                       float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes, void* stream) {
    moe_status_t st = validate_route(x, x_dt, T, H, w_router, E, k, score);
    if (st) return st;
    if (!routed) return fail(MOE_ERR_INVALID, "layer: null routed bank");
    const int I = routed->I;
    if (I <= 0 || I % 128) return fail(MOE_ERR_UNSUPPORTED, "layer: I=%d not a multiple of 128", I);
    if ((st = check_bank(routed, E, H, I, "routed"))) return st;
    if (shared && (st = check_bank(shared, 1, H, I, "shared"))) return st;
    const int wdt = routed->dt;
    if (shared && shared->dt != wdt) return fail(MOE_ERR_UNSUPPORTED, "layer: shared/routed dtype differ");
    const bool ok_combo = (x_dt == MOE_F32 && wdt == MOE_F32) ||
                          (x_dt == MOE_BF16 && (wdt == MOE_BF16 || wdt == MOE_E4M3 || wdt == MOE_MXFP4));
    if (!ok_combo) return fail(MOE_ERR_UNSUPPORTED, "layer: x dtype %d with weights %d", x_dt, wdt);
    if (out_dt != MOE_F32 && out_dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "layer: out dtype %d", out_dt);
    if (y_dt != MOE_F32 && y_dt != MOE_BF16 && y_dt != MOE_E4M3) return fail(MOE_ERR_UNSUPPORTED, "layer: y dtype %d", y_dt);
    if ((long long)T * k > (1LL << 30)) return fail(MOE_ERR_UNSUPPORTED, "layer: T*k too large");
    if (y_dt == MOE_E4M3 &&
        (wdt != MOE_E4M3 || !moe::gffn_e4m3_y_supported(H, I, T * k, shared ? T : 0)))
        return fail(MOE_ERR_UNSUPPORTED,
                    "layer: E4M3 y needs E4M3 weights, H %% 256 == 0 and row offsets within 32 bits "
                    "(H=%d I=%d T*k=%lld)", H, I, (long long)T * k);
    if (T == 0) return MOE_OK;
    if (!out || !aligned16(out) || !aligned16(x)) return fail(MOE_ERR_INVALID, "layer: null or misaligned x/out");
    const int has_sh = shared ? 1 : 0;
    const LayerWs L = layer_ws(T, H, E, k, I, x_dt, wdt, has_sh, out_dt, y_dt);
    if (!ws || ws_bytes < L.total || ((uintptr_t)ws & 255u)) return fail(MOE_ERR_WORKSPACE, "layer: workspace");
    uint8_t* w8 = (uint8_t*)ws;
    hipStream_t s = (hipStream_t)stream;
    const int R = T * k;
    int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(w8 + L.ids);
    float* tw = topk_w_out ? topk_w_out : (float*)(w8 + L.w);
    int32_t* counts = counts_out ? counts_out : (int32_t*)(w8 + L.counts);
    int32_t* offsets = (int32_t*)(w8 + L.offsets);
    int32_t* src = (int32_t*)(w8 + L.src);
    int32_t* dest = (int32_t*)(w8 + L.dest);
    const int ybf = out_dt == MOE_BF16;

    hipError_t e = moe::launch_router_logits(x, x_dt == MOE_BF16, T, H, w_router, bias, E, (float*)(w8 + L.logits), s);
    if (e == hipSuccess) e = moe::launch_router_topk((float*)(w8 + L.logits), T, E, k, score == MOE_SIGMOID, ids, tw, s);
    if (e == hipSuccess) e = moe::launch_permute(ids, R, E, counts, offsets, src, dest, w8 + L.perm, s);
    const void* a = x;
    const float* as = nullptr;
    if (e == hipSuccess && wdt == MOE_E4M3) {
        e = moe::launch_quant_e4m3(x, 1, T, H, w8 + L.xq, (float*)(w8 + L.xs), s);
        a = w8 + L.xq;
        as = (const float*)(w8 + L.xs);
    } else if (e == hipSuccess && wdt == MOE_MXFP4) {
        e = moe::launch_quant_mxfp8(x, 1, T, H, w8 + L.xq, w8 + L.xs, s);
        a = w8 + L.xq;
        as = (const float*)(w8 + L.xs);   // E8M0 bytes [T][H/32]
    }
    if (e == hipSuccess) {
        moe::GffnProblem p{};
        p.dt = wdt; p.a = a; p.a_scale = as; p.src = src; p.src_div = k;
        p.offsets = offsets; p.G = E; p.R_max = R; p.routed = to_bank(routed);
        p.a_sh = a; p.a_sh_scale = as; p.S = has_sh ? T : 0; p.has_shared = has_sh; p.shared = to_bank(shared);
        p.m_max = T;   // the router picks k distinct experts per token
        p.H = H; p.I = I; p.y = w8 + L.yperm; p.y_sh = has_sh ? w8 + L.ysh : nullptr;
        p.y_bf16 = y_dt == MOE_BF16; p.y_e4m3 = y_dt == MOE_E4M3; p.y_scale = (float*)(w8 + L.yscale);
        p.y_sh_bf16 = ybf;
        e = moe::launch_gffn(p, w8 + L.gffn, s);
    }
    if (e == hipSuccess)
        e = moe::launch_combine(w8 + L.yperm, y_dt == MOE_E4M3 ? 2 : y_dt == MOE_BF16 ? 1 : 0,
                                (const float*)(w8 + L.yscale), has_sh ? w8 + L.ysh : nullptr, ybf, dest, tw, T, k, H,
                                out, out_dt == MOE_BF16, s);
    return hip_check(e, "moe_layer");
}

}  // extern "C"
