/*
 * gen.c -- host side of the seeded input generator (see gen_core.h for the
 * definition of every value).  Exported with plain C types so Python can call
 * it through ctypes; OpenMP splits long fills over threads, which does not
 * change any value because each one depends only on its own counter.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "gen_core.h"

uint64_t gen_splitmix64_output(uint64_t state, uint64_t n) { return gen_splitmix_at(state, n); }

uint64_t gen_state(uint64_t seed, uint32_t layer, uint32_t tensor) {
  return gen_stream_state(seed, layer, tensor);
}

double gen_log01_host(double u) { return gen_log01(u); }
double gen_cos2pi01_host(double v) { return gen_cos2pi01(v); }

/* value i (i in [idx0, idx0 + n)) of stream (seed, layer, tensor), double */
void gen_normal_f64(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t idx0, int64_t n,
                    double sigma, double* out) {
  uint64_t s = gen_stream_state(seed, layer, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = sigma * gen_normal_at(s, idx0 + (uint64_t)i);
}

void gen_normal_f32(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t idx0, int64_t n,
                    double sigma, float* out) {
  uint64_t s = gen_stream_state(seed, layer, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = gen_to_f32(sigma * gen_normal_at(s, idx0 + (uint64_t)i));
}

void gen_normal_bf16(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t idx0, int64_t n,
                     double sigma, uint16_t* out) {
  uint64_t s = gen_stream_state(seed, layer, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = gen_f32_to_bf16(gen_to_f32(sigma * gen_normal_at(s, idx0 + (uint64_t)i)));
}

/* Per-expert router bias with Zipf(s) rank weights scaled to `scale`:
 * expert e has rank e + 1, b[e] = scale * (e + 1)^(-s), rounded to fp32. */
void gen_zipf_bias(int32_t E, double s, double scale, float* out) {
  for (int32_t e = 0; e < E; ++e) out[e] = (float)(scale * pow((double)(e + 1), -s));
}
