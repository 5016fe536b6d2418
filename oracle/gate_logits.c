/*
 * CPU oracle -- test infrastructure only.  Nothing on the product path may
 * link or call this file; tests, the smoke check and the benchmark's CPU
 * baseline do.
 *
 * Gate logits in a fixed fp32 evaluation order.
 *
 * The gate scores every token against every expert before any routing
 * decision is taken (ES-MoE review, section 三 技术架构, 专家级卸载与处理:
 * placement is only known once the gating network has run).  The pages print
 * no formula; the reading taken is a linear gate, l[t,e] = sum_i x[t,i] *
 * Wg[i,e] (+ a per-expert workload bias), evaluated in fp32 as a sequential
 * sum over i with every product and every sum rounded to nearest even and no
 * fused multiply-add:
 *
 *     acc = 0;  for i in 0..d-1: acc = fl(acc + fl(x[t,i] * Wg[i,e]));
 *     l[t,e] = bias ? fl(acc + bias[e]) : acc
 *
 * A fixed order makes the top-k routing decision reproducible bit for bit.
 * Must be compiled with -ffp-contract=off and without -ffast-math.
 */
#include <stddef.h>

void oracle_gate_logits_f32(const float *x, const float *Wg, const float *bias,
                            long T, long d, long E, float *out) {
#pragma omp parallel for schedule(static)
    for (long t = 0; t < T; ++t) {
        float *acc = out + t * E;
        for (long e = 0; e < E; ++e) acc[e] = 0.0f;
        const float *xr = x + t * d;
        for (long i = 0; i < d; ++i) {
            const float xi = xr[i];
            const float *w = Wg + i * E;
            for (long e = 0; e < E; ++e) {
                float p = xi * w[e];
                acc[e] = acc[e] + p;
            }
        }
        if (bias)
            for (long e = 0; e < E; ++e) acc[e] = acc[e] + bias[e];
    }
}
