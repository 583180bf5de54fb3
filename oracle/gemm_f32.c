/*
 * gemm_f32.c -- the CPU oracle's matrix product, plain C, single-threaded.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by oracle/__init__.py, which only the test-suite, the
 * smoke check and the benchmark's CPU-baseline leg import.  It shares no code with the
 * GPU library.
 *
 * What it computes (the layer's product with fp32 accumulation, as the workload
 * descriptions state it: "fp32 accumulate"):
 *
 *     y[t][o] = fl32( ... fl32( fl32(a[t][0] * b[0][o]) + a[t][1] * b[1][o] ) ... )
 *
 * i.e. for every output one fp32 accumulator that starts at +0 and adds the products in
 * ascending k, every product and every sum rounded to nearest even in fp32.  The operands
 * come from bf16 (8 significant bits) or e4m3 (4 bits) values, so every product is exact
 * in fp32 and only the sums round.  No fused multiply-add contraction and no
 * reassociation: the file is compiled with -ffp-contract=off and without -ffast-math.
 *
 * Loop order: the k loop sits outside the o loop, so the accumulators of one token row
 * (acc[0..o)) are advanced together one k at a time; each accumulator still sees its
 * products in ascending k, so this is the same arithmetic as the textbook t-o-k loop,
 * only with the weights read K-major (b[k][o]) so that a row of them is contiguous.
 */
#include <stdint.h>
#include <string.h>

/* a: fp32 [t][k] row-major; bk: fp32 [k][o] row-major (K-major weights); y: fp32 [t][o] */
void oracle_gemm_f32(const float* a, int64_t t, int64_t k, const float* bk, int64_t o, float* y) {
  for (int64_t i = 0; i < t; ++i) {
    float* acc = y + i * o;
    for (int64_t j = 0; j < o; ++j) acc[j] = 0.0f;
    for (int64_t kk = 0; kk < k; ++kk) {
      const float av = a[i * k + kk];
      const float* brow = bk + kk * o;
      for (int64_t j = 0; j < o; ++j) {
        const float p = av * brow[j];   /* exact for bf16 / e4m3 operands */
        acc[j] = acc[j] + p;            /* one fp32 rounding, ascending k */
      }
    }
  }
}
