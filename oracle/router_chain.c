/* Oracle: router logits in fp32, one fused multiply-add chain per logit.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is part of the CPU oracle: only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code with the GPU library.
 *
 * The router scores every token against every routed expert ("How DeepSeek
 * inference works", section "What does DeepSeek inference actually do per
 * token?": a learned router picks a small subset of experts per token;
 * "DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1, the "Gate:
 * router gate" operator).  The pages do not fix the precision or the order of
 * the dot product.  Because the chosen expert ids must be identical on the
 * CPU and on the GPU, the logit is defined here as a single fp32 chain:
 *
 *     acc = +0;  for h = 0 .. H-1 ascending:  acc = fmaf(x[t][h], Wr[h][e], acc)
 *     l[t][e] = acc + b[e]        (b[e] = +0 when there is no bias)
 *
 * The final addition of +0 turns a -0 sum into +0.  Built with
 * -ffp-contract=off so the compiler adds no contraction of its own; fmaf is
 * the correctly rounded fused multiply-add of C99.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* x: [T][H] fp32 (bf16 inputs are widened exactly by the caller)
 * wr: [H][E] fp32, b: [E] fp32 or NULL, l: [T][E] fp32 out. */
void oracle_router_logits(const float* x, int64_t T, int64_t H, const float* wr,
                          const float* b, int64_t E, float* l)
{
    for (int64_t t = 0; t < T; ++t) {
        float* acc = l + t * E;
        for (int64_t e = 0; e < E; ++e) acc[e] = 0.0f;
        const float* xt = x + t * H;
        for (int64_t h = 0; h < H; ++h) {
            const float xv = xt[h];
            const float* w = wr + h * E;
            /* independent chains over e; each chain runs over h in order */
            for (int64_t e = 0; e < E; ++e) acc[e] = fmaf(xv, w[e], acc[e]);
        }
        for (int64_t e = 0; e < E; ++e) acc[e] = acc[e] + (b ? b[e] : 0.0f);
    }
}
