/*
 * Seeded synthetic inputs for the layer-boundary workloads.
 *
 * This file is shared by both sides of every parity check (the HIP library
 * and the fp64 oracle receive the same bytes), so it holds none of the
 * boundary's own arithmetic: no sums of contributions, no residual update,
 * no normalisation and no output rounding. It only draws numbers.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: draw n
 * of stream (seed, id) is mix64(s0 + (n+1)*GOLDEN) with s0 a hash of
 * (seed, id). Every element is therefore a pure function of
 * (seed, id, index) and any slice can be regenerated on its own, in any
 * order, by any number of threads.
 *
 * Normals: Box-Muller (G. Box, M. Muller, 1958), cosine branch only;
 * normal number i uses draws 2i and 2i+1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t stream_origin(uint64_t seed, uint64_t id) {
  return mix64(mix64(seed + GOLDEN) ^ (id * 0xD1B54A32D192ED03ULL));
}

static uint64_t draw(uint64_t s0, uint64_t n) { return mix64(s0 + (n + 1) * GOLDEN); }

/* uniform in [0, 1) with 53 random bits */
static double unit_open_hi(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }
/* uniform in (0, 1] with 53 random bits */
static double unit_open_lo(uint64_t r) { return (double)((r >> 11) + 1) * 0x1.0p-53; }

static double normal_at(uint64_t s0, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unit_open_lo(draw(s0, 2 * i));
  double u2 = unit_open_hi(draw(s0, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* out[i] = (float)(mean + std * N_{first+i}) for i < count */
void gen_normal_f32(uint64_t seed, uint64_t id, uint64_t first, int64_t count, double mean,
                    double std, float* out) {
  const uint64_t s0 = stream_origin(seed, id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)(mean + std * normal_at(s0, first + (uint64_t)i));
}

/* out[i] = U_{first+i}, uniform in [0, 1) */
void gen_uniform_f64(uint64_t seed, uint64_t id, uint64_t first, int64_t count, double* out) {
  const uint64_t s0 = stream_origin(seed, id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = unit_open_hi(draw(s0, first + (uint64_t)i));
}

/*
 * Normals with sparse outliers: element i is mean + std*N_i, multiplied by
 * `factor` when the independent uniform U_i of stream `mask_id` is below
 * `prob`. Values are produced in float before any rounding to bf16.
 */
void gen_outlier_normal_f32(uint64_t seed, uint64_t id, uint64_t mask_id, uint64_t first,
                            int64_t count, double mean, double std, double prob, double factor,
                            float* out) {
  const uint64_t s0 = stream_origin(seed, id);
  const uint64_t m0 = stream_origin(seed, mask_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    double v = mean + std * normal_at(s0, first + (uint64_t)i);
    if (unit_open_hi(draw(m0, first + (uint64_t)i)) < prob) v *= factor;
    out[i] = (float)v;
  }
}

/*
 * Top-k routing for a MoE layer, used to lay out the expert-output buffer.
 *
 * Token t has n_experts router logits N(0,1) (normal numbers
 * t*n_experts .. t*n_experts+n_experts-1 of stream logits_id). Its k picks
 * are the k largest logits in descending order (ties: lower expert id
 * first). gate[t*k+j] is the softmax over the k picked logits, evaluated
 * in double and stored as float. expert[t*k+j] is the j-th picked expert.
 *
 * The expert-output rows are stored expert-major: all rows of expert 0,
 * then expert 1, ..., and within an expert ordered by (t, j). idx[t*k+j]
 * is the row of that buffer holding token t's j-th pick (gather form).
 *
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int gen_moe_routing(uint64_t seed, uint64_t logits_id, int64_t T, int n_experts, int k,
                    int32_t* idx, float* gate, int32_t* expert) {
  if (T < 0 || n_experts < 1 || k < 1 || k > n_experts) return -1;
  const uint64_t s0 = stream_origin(seed, logits_id);
  double* logit = (double*)malloc(sizeof(double) * (size_t)n_experts);
  unsigned char* taken = (unsigned char*)malloc((size_t)n_experts);
  int64_t* count = (int64_t*)calloc((size_t)n_experts, sizeof(int64_t));
  if (!logit || !taken || !count) {
    free(logit);
    free(taken);
    free(count);
    return -1;
  }
  for (int64_t t = 0; t < T; ++t) {
    for (int e = 0; e < n_experts; ++e) {
      logit[e] = normal_at(s0, (uint64_t)(t * n_experts + e));
      taken[e] = 0;
    }
    double pick_logit[64];
    double* pl = k <= 64 ? pick_logit : (double*)malloc(sizeof(double) * (size_t)k);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < n_experts; ++e)
        if (!taken[e] && (best < 0 || logit[e] > logit[best])) best = e;
      taken[best] = 1;
      expert[t * k + j] = best;
      pl[j] = logit[best];
      count[best]++;
    }
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(pl[j] - pl[0]);
    for (int j = 0; j < k; ++j) gate[t * k + j] = (float)(exp(pl[j] - pl[0]) / z);
    if (pl != pick_logit) free(pl);
  }
  /* expert-major placement, (t, j) ascending inside each expert */
  int64_t* next = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_experts);
  if (!next) {
    free(logit);
    free(taken);
    free(count);
    return -1;
  }
  int64_t base = 0;
  for (int e = 0; e < n_experts; ++e) {
    next[e] = base;
    base += count[e];
  }
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) idx[t * k + j] = (int32_t)(next[expert[t * k + j]]++);
  free(next);
  free(logit);
  free(taken);
  free(count);
  return 0;
}
