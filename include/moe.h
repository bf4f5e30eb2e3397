/* moe.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN layer.
 *
 * The layer follows the DeepSeek-style MoE FFN the pages describe:
 *   route    -> a learned router scores every token against E routed experts
 *               and keeps the top k ("How DeepSeek inference works", section
 *               "What does DeepSeek inference actually do per token?" and its
 *               worked example of 256 experts with 8 active per token;
 *               "DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1,
 *               operator "Gate: router gate & prepare shared GEMM");
 *   permute  -> the T*k token-expert assignments are grouped by expert
 *               (same page, section 2.3.1, "Expert: prepare routed GEMM");
 *   grouped FFN -> per expert, h = silu(x W_gate) * (x W_up) ("up & gate",
 *               one [7168, 4096] = [H, 2I] product, then "SwiGLU") and
 *               y = h W_down ("down", [2048, 7168] = [I, H]); the shared
 *               expert runs on every token (section 2.3.1, "Shared expert
 *               GEMM"; section 2.4.1 for the decode shapes);
 *   combine  -> out[t] = y_shared[t] + sum_j w[t][j] * y[t, expert j]
 *               (section 2.3.1, "Expert: combine reduce").
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, allocated and owned by the
 *    caller; moe_experts_t is a host struct holding device pointers and is
 *    read only during the call.  The library never allocates or frees device
 *    memory: scratch comes from the caller's workspace `ws` (at least the
 *    size the matching *_workspace_size query returns; 256-byte aligned).
 *  - Calls only enqueue kernels on `stream` (a hipStream_t; NULL is the
 *    default stream) and return; there is no host synchronisation and no
 *    device-to-host copy (per-expert counts stay on the device).
 *  - Arguments are validated before anything is launched: MOE_ERR_INVALID
 *    (bad size, null required pointer), MOE_ERR_UNSUPPORTED (dtype
 *    combination or size the kernels do not implement), MOE_ERR_WORKSPACE
 *    (ws_bytes too small).  A failed launch gives MOE_ERR_HIP.  The text of
 *    the last error of the calling thread is available from moe_last_error().
 *    T = 0 (or R = 0) is a valid no-op.
 *  - Inputs containing NaN or Inf are a precondition violation (unchecked).
 *  - Results are bitwise deterministic from run to run (no floating-point
 *    atomics).  Thread-safe: no mutable global state except the per-thread
 *    error text.
 *  - Matrices are row-major.  Expert weights are stored OUTPUT-MAJOR (the
 *    reduction index contiguous, like a linear layer's [out][in] weight):
 *        w_gate, w_up : [n][I][H]   element (h, i) of W_gate (H x I) at [e][i][h]
 *        w_down       : [n][H][I]   element (i, c) of W_down (I x H) at [e][c][i]
 *    E4M3 banks carry one fp32 scale per 128 x 128 block, in the same order:
 *        s_gate, s_up : [n][I/128][H/128],  s_down : [n][H/128][I/128]
 *    and the represented weight is e4m3_value(code) * scale.
 *    MXFP4 banks (OCP Microscaling FP4: E2M1 elements, one E8M0 exponent per
 *    32 consecutive reduction elements) pack two codes per byte along the
 *    reduction index, the lower index in the low nibble, and carry one
 *    exponent byte per 32 elements, in the same order:
 *        w_gate, w_up : [n][I][H/2] bytes,  s_gate, s_up : [n][I][H/32] bytes
 *        w_down       : [n][H][I/2] bytes,  s_down       : [n][H][I/32] bytes
 *    The represented weight is e2m1_value(code) * 2^(E - 127).
 *  - E4M3 means OCP FP8 E4M3FN (bias 7, max 448, no infinities).  MXFP8
 *    activations are E4M3 codes [rows][cols] with one E8M0 byte per row and
 *    32 columns [rows][cols/32] (OCP Microscaling), produced by
 *    moe_quant_mxfp8; E2M1 is 1 sign, 2 exponent (bias 1), 1 mantissa bit:
 *    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2, MOE_MXFP4 = 3, MOE_MXFP8 = 4 } moe_dtype_t;

typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score_t;

/* A bank of n experts (the shared expert is a bank with n = 1).  dt is the
 * weight type: MOE_F32, MOE_BF16, MOE_E4M3 (fp32 block scales s_* required)
 * or MOE_MXFP4 (E8M0 exponent bytes s_* required).  H and I are the logical
 * sizes (elements) and must be multiples of 128 for every dtype. */
typedef struct {
    int32_t n, H, I;
    int32_t dt;                 /* moe_dtype_t */
    const void* w_gate;         /* [n][I][H]   (MXFP4: [n][I][H/2] bytes) */
    const void* w_up;           /* [n][I][H]   (MXFP4: [n][I][H/2] bytes) */
    const void* w_down;         /* [n][H][I]   (MXFP4: [n][H][I/2] bytes) */
    const void* s_gate;         /* E4M3: fp32 [n][I/128][H/128]; MXFP4: uint8 [n][I][H/32] */
    const void* s_up;           /* E4M3: fp32 [n][I/128][H/128]; MXFP4: uint8 [n][I][H/32] */
    const void* s_down;         /* E4M3: fp32 [n][H/128][I/128]; MXFP4: uint8 [n][H][I/32] */
    /* MXFP4 only, optional (NULL: unused; s_* stay required): the same
     * exponents in the order the 16-row MXFP4 streaming tiles read them,
     * written by moe_mx_pack_scales.  Used when the routed bank and (if
     * present) the shared bank both carry them. */
    const void* s_gate_up_packed;   /* uint8 [n][I/32][H/512][64][16] */
    const void* s_down_packed;      /* uint8 [n][H/64][I/512][64][16] */
} moe_experts_t;

/* ---- routing ("How DeepSeek inference works", "What does DeepSeek inference
 * actually do per token?": a learned router scores the routed experts and keeps
 * the top k, 8 of 256 in its worked example; "DeepSeek V3/R1 Inference
 * Efficiency (2)", section 2.3.1, operator "Gate: router gate") -------------
 * For every token t and routed expert e the logit is one fp32 chain of fused
 * multiply-adds over h = 0..H-1 in ascending order,
 *     l[t][e] = fma-chain(x[t][h] * w_router[h][e]) + bias[e]   (+0 adds turn -0 into +0),
 * so the result is independent of the launch shape.  The k experts with the
 * largest logits are kept in descending order (equal logits: lower expert
 * index first).  Weights over the k chosen, in double precision, stored fp32:
 *     MOE_SOFTMAX: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *     MOE_SIGMOID: w_j = s_j / sum_i s_i,   s_j = 1 / (1 + exp(-l_j))
 * x: [T][H], x_dt MOE_F32 or MOE_BF16; w_router: [H][E] fp32; bias: [E] fp32
 * or NULL; 1 <= k <= E <= 1024; H % 128 == 0.
 * Outputs: topk_ids [T][k] int32, topk_w [T][k] fp32. */
moe_status_t moe_route(const void* x, int32_t x_dt, int32_t T, int32_t H,
                       const float* w_router, const float* bias, int32_t E, int32_t k,
                       int32_t score, int32_t* topk_ids, float* topk_w,
                       void* ws, size_t ws_bytes, void* stream);
size_t moe_route_workspace_size(int32_t T, int32_t E);

/* ---- permute ("DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1,
 * operator "Expert: prepare routed GEMM": token-expert assignments gathered
 * per expert before the grouped GEMM) ---------------------------------------
 * Groups the R = T*k assignments by expert (stable counting sort):
 *   counts[e]   number of assignments to expert e                 [E]
 *   offsets     exclusive prefix sum of counts, offsets[E] = R    [E+1]
 *   src[p]      flat assignment index f = t*k + j at permuted
 *               position p; ascending f within an expert          [R]
 *   dest[f]     permuted position of assignment f                 [R]
 * topk_ids: [T][k] int32 with values in [0, E); 1 <= E <= 1024. */
moe_status_t moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                         int32_t* counts, int32_t* offsets, int32_t* src, int32_t* dest,
                         void* ws, size_t ws_bytes, void* stream);
/* 0 for invalid sizes, including T * k > 2^30. */
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E);

/* ---- activation quantisation (the BF16 -> FP8 cast of section 2.3.1) ------
 * Per row and per block of 128 columns: amax = max|v|; scale = amax / 448 as
 * an IEEE fp32 division (1 when amax == 0); q = e4m3(v / scale) with an IEEE
 * fp32 division, rounding to nearest even and saturating at 448 (the sign
 * of v is kept, so a negative value that rounds to zero gives code 0x80).
 * x: [rows][cols] MOE_F32 or MOE_BF16, cols % 128 == 0.
 * Outputs: q [rows][cols] uint8 codes, scale [rows][cols/128] fp32. */
moe_status_t moe_quant_e4m3_1x128(const void* x, int32_t x_dt, int32_t rows, int32_t cols,
                                  uint8_t* q, float* scale, void* stream);

/* ---- MXFP8 activation quantisation (OCP Microscaling; the activation
 * format of the MXFP4 expert GEMMs, the FP4 MoE of the pages' Blackwell
 * deployment: "How DeepSeek inference works", deployment lever table) -------
 * Per row and block of 32 columns: E = clamp(floor(log2(amax)) - 8 + 127,
 * 0, 254) (E = 0 for an all-zero block), then q = e4m3(v * 2^(127 - E)) with
 * the product exact, rounding to nearest even and saturating at 448.
 * x: [rows][cols] MOE_F32 or MOE_BF16, cols % 32 == 0.
 * Outputs: q [rows][cols] uint8 E4M3 codes, e8m0 [rows][cols/32] uint8. */
moe_status_t moe_quant_mxfp8(const void* x, int32_t x_dt, int32_t rows, int32_t cols,
                             uint8_t* q, uint8_t* e8m0, void* stream);

/* ---- grouped FFN ("DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1:
 * routed "up & gate" [7168, 4096] and "down" [2048, 7168] grouped GEMMs with
 * "Expert: SwiGLU" between them, and the shared expert GEMMs; section 2.4.1 for
 * the decode sizes; section 1.b for efficiency against group count and rows
 * per group) ----------------------------------------------------------------
 * For every routed group g (expert g of `routed`) and permuted row p in
 * [offsets[g], offsets[g+1]):
 *     a_p = a[src[p] / src_div]   (a[p] when src is NULL; src values in [0, R_max))
 *     h_p = silu(a_p W_gate) * (a_p W_up),   silu(z) = z / (1 + exp(-z))
 *     y[p] = round_y(h'_p W_down)
 * and, when `shared` is non-NULL, the same with the shared expert for the S
 * rows of a_sh into y_sh.  h' is h at the precision the down projection
 * consumes: F32 weights -> fp32; BF16 -> rounded to bf16 (nearest even);
 * E4M3 -> quantised per row and 128-column block from its fp32 value by the
 * rule of moe_quant_e4m3_1x128 (scale = amax / 448 and codes = h / scale, both
 * IEEE fp32 divisions); MXFP4 -> MXFP8 per row and 32 columns by the rule of
 * moe_quant_mxfp8.  The fp32 value of h itself depends on the accumulation
 * order, so h's codes equal those of a reference only up to that rounding.
 * Accumulation is fp32.
 * Supported (a_dt, weight dt): (F32, F32), (BF16, BF16), (E4M3, E4M3),
 * (MXFP8, MXFP4).  E4M3 activations carry fp32 a_scale [rows of a][H/128],
 * MXFP8 activations uint8 a_scale [rows of a][H/32] (a_sh_scale likewise).
 * offsets: [G+1] int32 device array with offsets[0] = 0 and
 * offsets[G] <= R_max (R_max, a host value, bounds the routed rows and sizes
 * the launch).  y: [R_max][H] of type y_dt: F32, BF16, or E4M3 = codes
 * quantised per row and 128-column block by the rule of moe_quant_e4m3_1x128
 * from the fp32 accumulators, with the scales in y_scale [R_max][H/128]
 * (E4M3 y needs E4M3 weights, H a multiple of 256, and max(R_max, S) * H and
 * (R_max + S) * I below 2^32, else MOE_ERR_UNSUPPORTED; y_scale is ignored
 * otherwise).  y_sh: [S][H] of type y_sh_dt (F32 or BF16).
 * routed->n must equal G; H, I multiples of 128.  A call with rows to
 * process needs G >= 1 (the shared expert alone, G = 0, returns
 * MOE_ERR_UNSUPPORTED) and a non-NULL offsets array. */
moe_status_t moe_grouped_ffn(const void* a, int32_t a_dt, const void* a_scale,
                             const int32_t* src, int32_t src_div,
                             const int32_t* offsets, int32_t G, int32_t R_max,
                             const moe_experts_t* routed,
                             const void* a_sh, const void* a_sh_scale, int32_t S,
                             const moe_experts_t* shared,
                             void* y, int32_t y_dt, float* y_scale, void* y_sh, int32_t y_sh_dt,
                             void* ws, size_t ws_bytes, void* stream);
size_t moe_grouped_ffn_workspace_size(int32_t R_max, int32_t G, int32_t S, int32_t H,
                                      int32_t I, int32_t w_dt);

/* ---- packed MXFP4 exponents (for MXFP4 expert weights, the FP4 MoE GEMMs
 * of "How DeepSeek inference works", deployment lever table) --------------
 * A weight-load-time step, not part of the per-token path: writes the E8M0
 * exponents of an MXFP4 bank (s_gate, s_up [n][I][H/32], s_down [n][H][I/32])
 * again, permuted into the order in which the 16-row MXFP4 streaming tiles
 * consume them, so that one 16-byte load per lane brings exactly the
 * exponents the lane needs for four 128-wide k-steps of four weight blocks.
 * With c = lane / 16 (32-wide K block within a step), r = lane % 16 (row in
 * a 16-row weight block), q = 4 ss + b (ss: step within the group of four,
 * b: block):
 *   s_gate_up_packed[e][i32][j][lane][q] = (b < 2 ? s_gate : s_up)
 *       [e][32 i32 + 16 (b % 2) + r][4 (4 j + ss) + c]
 *   s_down_packed[e][h64][j][lane][q] = s_down[e][64 h64 + 16 b + r][4 (4 j + ss) + c]
 * Sizes: 2 n I (H/32) and n H (I/32) bytes, 16-byte aligned, owned by the
 * caller.  Requires dt == MOE_MXFP4 with H % 1024 == 0 and I % 512 == 0
 * (MOE_ERR_UNSUPPORTED otherwise); a bank is not modified.  Either output
 * may be NULL (not written).  Enqueued on `stream`.  A bank carrying the
 * packed exponents gives results identical to the same bank without them. */
moe_status_t moe_mx_pack_scales(const moe_experts_t* bank, void* s_gate_up_packed, void* s_down_packed,
                                void* stream);

/* ---- combine ------------------------------------------------------------
 * out[t] = y_sh[t] + sum_{j=0}^{k-1} topk_w[t][j] * y_perm[dest[t*k+j]]
 * accumulated in fp32 in this order (y_sh = 0 when NULL), then rounded to
 * out_dt (F32 or BF16).  y_perm: [T*k][H] of type y_dt (F32, BF16, or E4M3
 * codes whose value is code * y_scale[row][col/128], y_scale [T*k][H/128]:
 * the FP8 combine of "DeepSeek V3/R1 Inference Efficiency (2)", section 2);
 * y_sh: [T][H] of type y_sh_dt (F32 or BF16). */
moe_status_t moe_combine(const void* y_perm, int32_t y_dt, const float* y_scale,
                         const void* y_sh, int32_t y_sh_dt,
                         const int32_t* dest, const float* topk_w, int32_t T, int32_t k,
                         int32_t H, void* out, int32_t out_dt, void* stream);

/* ---- the whole layer (the MoE FFN of "How DeepSeek inference works" and of
 * "DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1: gate, prepare
 * routed GEMM, routed and shared expert GEMMs with SwiGLU, combine reduce) ---
 * route -> (E4M3 or MXFP4 weights: quantise x once per token, per 1x128
 * block or to MXFP8) -> permute -> grouped FFN over the routed groups and
 * the shared expert -> combine, all enqueued on `stream`.  Supported: x F32
 * with F32 weights; x BF16 with BF16, E4M3 or MXFP4 weights.  y_sh is kept in fp32 when out_dt is F32 and in bf16 when out_dt
 * is BF16; the routed expert outputs y_perm in y_dt: F32 or BF16, or E4M3
 * (the FP8 combine; E4M3 weights, H a multiple of 256, T*k*H and
 * (T*k + T)*I below 2^32 only, else MOE_ERR_UNSUPPORTED).
 * topk_ids_out [T][k], topk_w_out [T][k], counts_out [E] are optional copies
 * of the routing results (NULL to skip). */
moe_status_t moe_layer(const void* x, int32_t x_dt, int32_t T, int32_t H,
                       const float* w_router, const float* bias, int32_t E, int32_t k,
                       int32_t score, const moe_experts_t* routed, const moe_experts_t* shared,
                       void* out, int32_t out_dt, int32_t y_dt,
                       int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                       void* ws, size_t ws_bytes, void* stream);
size_t moe_layer_workspace_size(int32_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                                int32_t x_dt, int32_t w_dt, int32_t has_shared, int32_t out_dt,
                                int32_t y_dt);

/* ---- the whole layer without a workspace --------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): moe_layer
 * with the same arguments and results, whose scratch is a 64 MiB device array
 * inside the library (one per GPU, held until the process ends) instead of
 * a caller workspace.  No allocation happens in the call.
 *  - Calls needing more scratch than the array (moe_layer_workspace_size of
 *    their sizes above 64 MiB; for the 7168 x 2048 x 256-expert layer with
 *    bf16 weights: T above 400 with bf16 outputs, above 226 with fp32
 *    outputs) return MOE_ERR_UNSUPPORTED before any launch.
 *  - The array of a GPU is shared by every call on it and keeps the last
 *    call's contents; nothing in it needs to start at zero (each call writes
 *    every scratch value it reads).  Calls that overlap on one GPU (two host
 *    threads, or two streams whose work runs concurrently) race on it and
 *    give undefined results: order them on one stream or with events.
 *  - `stream` must belong to the current device (else MOE_ERR_INVALID); the
 *    array's address is looked up on the first call on each device. */
moe_status_t moe_layer_noalloc(const void* x, int32_t x_dt, int32_t T, int32_t H,
                               const float* w_router, const float* bias, int32_t E, int32_t k,
                               int32_t score, const moe_experts_t* routed, const moe_experts_t* shared,
                               void* out, int32_t out_dt, int32_t y_dt,
                               int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                               void* stream);

/* Name of a status code; text of the calling thread's last error ("" if none). */
const char* moe_status_string(int32_t status);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
