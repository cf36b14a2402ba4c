/*
 * ds4gen_host.c -- host side of the synthetic input generator (C ABI, used
 * through ctypes).  See ds4gen.h for the random stream.  Everything here is
 * input construction: random draws, their distributions, and rounding of the
 * drawn values to the storage formats the inputs are specified in.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -o libds4gen.so ds4gen_host.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "ds4gen.h"

#define EXPORT __attribute__((visibility("default")))

/* Raw blocks [first, first+n) of a quantised tensor stream. */
EXPORT void ds4gen_blocks(int qtype, uint64_t seed, uint64_t stream, uint64_t first,
                          uint64_t n, uint8_t* out) {
  uint64_t key = gen_key(seed, stream);
  int bb = gen_block_bytes(qtype);
  for (uint64_t i = 0; i < n; i++) gen_block(qtype, key, first + i, out + i * (uint64_t)bb);
}

/* The 256 x 8 grid: each entry one of {8, 25, 43}, chosen uniformly. */
EXPORT void ds4gen_grid(uint64_t seed, uint8_t* out) {
  static const uint8_t vals[3] = {8, 25, 43};
  uint64_t key = gen_key(seed, DS4GEN_GRID);
  for (int i = 0; i < 256 * 8; i++) out[i] = vals[gen_below(gen_draw(key, (uint64_t)i), 3u)];
}

/* Standard normal deviate number i of a stream (Box-Muller on draws 2i, 2i+1). */
static double normal_at(uint64_t key, uint64_t i) {
  uint64_t d1 = gen_draw(key, 2 * i), d2 = gen_draw(key, 2 * i + 1);
  double u1 = ((double)(d1 >> 11) + 1.0) * 0x1.0p-53; /* (0,1] */
  double u2 = (double)(d2 >> 11) * 0x1.0p-53;         /* [0,1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

EXPORT void ds4gen_normal_f64(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                              double mean, double std, double* out) {
  uint64_t key = gen_key(seed, stream);
  for (uint64_t i = 0; i < n; i++) out[i] = mean + std * normal_at(key, first + i);
}

/* N(mean, std^2) rounded to fp16 / bf16 / fp32 storage. */
EXPORT void ds4gen_normal_f16(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                              double mean, double std, uint16_t* out) {
  uint64_t key = gen_key(seed, stream);
  for (uint64_t i = 0; i < n; i++) out[i] = gen_f16(mean + std * normal_at(key, first + i));
}
EXPORT void ds4gen_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                               double mean, double std, uint16_t* out) {
  uint64_t key = gen_key(seed, stream);
  for (uint64_t i = 0; i < n; i++) out[i] = gen_bf16(mean + std * normal_at(key, first + i));
}
EXPORT void ds4gen_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                              double mean, double std, float* out) {
  uint64_t key = gen_key(seed, stream);
  for (uint64_t i = 0; i < n; i++) out[i] = (float)(mean + std * normal_at(key, first + i));
}

/* U[a,b) rounded to fp32. */
EXPORT void ds4gen_uniform_f32(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                               double a, double b, float* out) {
  uint64_t key = gen_key(seed, stream);
  for (uint64_t i = 0; i < n; i++) out[i] = (float)gen_uniform(gen_draw(key, first + i), a, b);
}

/* Integers uniform in [0, bound). */
EXPORT void ds4gen_uniform_int(uint64_t seed, uint64_t stream, uint64_t first, uint64_t n,
                               uint32_t bound, int32_t* out) {
  uint64_t key = gen_key(seed, stream);
  for (uint64_t i = 0; i < n; i++) out[i] = (int32_t)gen_below(gen_draw(key, first + i), bound);
}

/*
 * Correlated token activations: row t = bf16(alpha * c + beta * n_t), with c
 * one shared N(0,1) vector (stream_c) and n_t independent N(0,1) rows
 * (stream_n).  alpha^2 + beta^2 = 1 keeps unit variance.
 */
EXPORT void ds4gen_mixed_bf16(uint64_t seed, uint64_t stream_c, uint64_t stream_n, int64_t T,
                              int64_t H, double alpha, double beta, uint16_t* out) {
  uint64_t kc = gen_key(seed, stream_c), kn = gen_key(seed, stream_n);
  for (int64_t t = 0; t < T; t++)
    for (int64_t c = 0; c < H; c++) {
      double a = alpha * normal_at(kc, (uint64_t)c);
      double b = beta * normal_at(kn, (uint64_t)(t * H + c));
      out[t * H + c] = gen_bf16(a + b);
    }
}

/*
 * Hash-routing table rows [first_tok, first_tok+n_tok): for each token K
 * distinct expert ids in [0,E), drawn uniformly with rejection of repeats
 * (draw indices 64*tok + j).  Returns the number of rows that failed to
 * find K distinct ids within 64 draws (never expected; 0 on success).
 */
EXPORT int ds4gen_tid2eid(uint64_t seed, uint64_t stream, int64_t first_tok, int64_t n_tok,
                          int E, int K, int32_t* out) {
  uint64_t key = gen_key(seed, stream);
  int fails = 0;
  for (int64_t t = 0; t < n_tok; t++) {
    int32_t* row = out + t * K;
    int got = 0;
    for (int j = 0; j < 64 && got < K; j++) {
      int32_t e = (int32_t)gen_below(gen_draw(key, (uint64_t)(first_tok + t) * 64ULL + j), (uint32_t)E);
      int dup = 0;
      for (int q = 0; q < got; q++) dup |= (row[q] == e);
      if (!dup) row[got++] = e;
    }
    if (got < K) fails++;
  }
  return fails;
}

/*
 * Caller-given routing with Zipf-skewed expert load (prefill workload):
 *  - a uniformly random ranking of the E experts (Fisher-Yates on stream
 *    RANKPERM); the expert at rank r (1-based) has popularity p_r = r^-s;
 *  - each token picks K distinct experts by sampling without replacement
 *    proportionally to p (Gumbel-top-K: the K largest log p + G, G Gumbel);
 *  - gate weights u_k ~ U(0,1], normalised so each token's K weights sum
 *    to `total` (1.5), stored as fp32.
 */
EXPORT void ds4gen_zipf_routing(uint64_t seed, int T, int E, int K, double s, double total,
                                int32_t* ids, float* gates) {
  uint64_t kp = gen_key(seed, DS4GEN_RANKPERM), kr = gen_key(seed, DS4GEN_ROUTE),
           kg = gen_key(seed, DS4GEN_GATES);
  int* rank_of = (int*)malloc(sizeof(int) * E);
  int* order = (int*)malloc(sizeof(int) * E);
  double* key = (double*)malloc(sizeof(double) * E);
  for (int i = 0; i < E; i++) order[i] = i;
  for (int i = E - 1; i > 0; i--) {
    int j = (int)gen_below(gen_draw(kp, (uint64_t)i), (uint32_t)(i + 1));
    int tmp = order[i];
    order[i] = order[j];
    order[j] = tmp;
  }
  for (int r = 0; r < E; r++) rank_of[order[r]] = r + 1;
  for (int t = 0; t < T; t++) {
    for (int e = 0; e < E; e++) {
      double u = ((double)(gen_draw(kr, (uint64_t)t * E + e) >> 11) + 0.5) * 0x1.0p-53;
      key[e] = -s * log((double)rank_of[e]) - log(-log(u));
    }
    for (int k = 0; k < K; k++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        int taken = 0;
        for (int q = 0; q < k; q++) taken |= (ids[t * K + q] == e);
        if (taken) continue;
        if (best < 0 || key[e] > key[best]) best = e;
      }
      ids[t * K + k] = best;
    }
    double u[64], sum = 0.0;
    for (int k = 0; k < K && k < 64; k++) {
      u[k] = ((double)(gen_draw(kg, (uint64_t)t * K + k) >> 11) + 1.0) * 0x1.0p-53;
      sum += u[k];
    }
    for (int k = 0; k < K && k < 64; k++) gates[t * K + k] = (float)(total * u[k] / sum);
  }
  free(rank_of);
  free(order);
  free(key);
}
