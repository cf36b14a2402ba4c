/*
 * ds4_encode.c -- plain CPU reference of the block encoders (float matrix ->
 * Q2_K / IQ2_XXS blocks), with and without per-column importance weights.
 * TEST INFRASTRUCTURE ONLY, part of liboracle.so like ds4_oracle.c: the test
 * suite and the benchmark's CPU-baseline leg call it; the GPU library never
 * does, and the two share no code.
 *
 * What the pages fix (DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec):
 *   sec. 3  Q2_K: a scale and a minimum are estimated per 16 values, values are
 *           rounded to 2-bit codes 0..3, four codes are packed per byte; with
 *           an importance vector a weighted variant changes how scales and
 *           codes are chosen (importance weighs the quantisation error).
 *   sec. 4  IQ2_XXS: 8 groups of 32 values, four 8-value grid indices and
 *           four 7-bit sign masks per group, fp16 block scale refined by a
 *           4-bit group nibble, a 256-entry grid; tuples not on the grid are
 *           searched in a nearest-neighbour list (two shells); the encoder
 *           requires an importance vector.
 *   sec. 5, 7, 8  importance[column] = sum of squared activations; one
 *           vector per expert (n_expert x n_columns); without measured
 *           statistics the fallback is the column energy of the weights.
 * The Q4 files of the mixed stacks (DS4C2 sec. 10) and the Q8_0 shared
 * experts (FLOW quantisation table) come from the same tool; their encoders
 * here are the plain readings: Q4_K = the Q2_K procedure on 32-value
 * sub-blocks with 4-bit codes and 6-bit scale/min nibbles; Q8_0 = d =
 * max|x| / 127 per 32 values, nearest codes.
 * The pages print no search procedure.  The one below is a plain reading
 * (every choice is written at the function): a fixed number of weighted
 * least-squares refits for Q2_K, a fixed set of candidate group scales for
 * IQ2_XXS.  Parity of these procedures is unpinned by the pages; the tests
 * pin them by exact round trips of representable blocks, brute force on
 * small cases and statistical properties.
 *
 * Precision: the encoders decide integers (codes, nibbles, grid indices) from
 * floating point, so every decision is taken in binary32 with the operation
 * order written here (sums run over the values in index order, one rounding
 * per operation, no contraction: the library builds with -ffp-contract=off),
 * so that another binary32 implementation of the same steps makes the same
 * decisions.  Division is IEEE division, rintf rounds half to even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

enum { EN_Q2_K = 0, EN_IQ2_XXS = 1, EN_Q8_0 = 2, EN_Q4_K = 3 };
enum { EN_OK = 0, EN_EINVAL = -1 };

/* binary32 -> binary16 bits, round to nearest even (subnormals kept,
 * overflow to infinity).  Exact: the binary32 value is exact in double. */
EXPORT uint16_t en_f16_bits(float f) {
  double v = (double)f;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(a)) return 0x7E00;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                    /* a = m 2^e, 0.5 <= m < 1 */
  int q = e - 11;                  /* 11 significant bits */
  if (q < -24) q = -24;            /* subnormal quantum 2^-24 */
  double r = ldexp(rint(ldexp(a, -q)), q);
  if (r == 0.0) return sign;               /* rounds to zero */
  if (r >= 65520.0) return sign | 0x7C00;  /* rounds past 65504 */
  frexp(r, &e);
  int E = e - 1 + 15;
  if (E >= 1) {
    int mant = (int)(ldexp(r, -(e - 1)) * 1024.0) - 1024;
    return sign | (uint16_t)(E << 10) | (uint16_t)mant;
  }
  return sign | (uint16_t)ldexp(r, 24);
}

static float f16_float(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v = e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
  return (float)(s ? -v : v);
}

static float clampf(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

/* ------------------------------------------------------------------ */
/* Q2_K                                                                */
/* ------------------------------------------------------------------ */

/* Code of x for scale s and min m: nearest of s*q - m, q in 0..qmax. */
static int af_code(float x, float s, float m, float qmax) {
  if (!(s > 0.0f)) return 0;
  return (int)clampf(rintf((x + m) / s), 0.0f, qmax);
}

/* Weighted squared error of the n values of a sub-block for (s, m). */
static float af_err(const float* x, const float* w, int n, float s, float m, float qmax) {
  float e = 0.0f;
  for (int i = 0; i < n; i++) {
    float t = s * (float)af_code(x[i], s, m, qmax);
    t = t - m;
    float r = t - x[i];
    e = e + w[i] * (r * r);
  }
  return e;
}
static int q2_code(float x, float s, float m) { return af_code(x, s, m, 3.0f); }

/*
 * Scale s >= 0 and min m >= 0 of one sub-block of n values for x ~ s*q - m,
 * q in 0..qmax (Q2_K: 16 values, qmax 3; Q4_K: 32 values, qmax 15).
 * Start: the range, m = -min(0, min x), s = (max x + m) / qmax (a sub-block whose
 * values are all equal and not positive is exact with s = 0).  Then four
 * rounds of: codes for the current (s, m), weighted least-squares (s, m) for
 * those codes (m clamped at 0, then s at 0), keeping the pair with the lowest
 * weighted error (strictly lower replaces; the start wins ties).
 */
static void af_fit(const float* x, const float* w, int n, float qmax, float* s_out,
                   float* m_out) {
  float lo = 0.0f, hi = x[0];
  for (int i = 0; i < n; i++) {
    lo = fminf(lo, x[i]);
    hi = fmaxf(hi, x[i]);
  }
  float s = (hi - lo) / qmax, m = -lo;
  if (!(s > 0.0f)) s = 0.0f;
  float bs = s, bm = m, be = af_err(x, w, n, s, m, qmax);
  for (int it = 0; it < 4; it++) {
    float S0 = 0.0f, S1 = 0.0f, S2 = 0.0f, T0 = 0.0f, T1 = 0.0f;
    for (int i = 0; i < n; i++) {
      float q = (float)af_code(x[i], s, m, qmax);
      float wq = w[i] * q;
      S0 = S0 + w[i];
      S1 = S1 + wq;
      S2 = S2 + wq * q;
      T0 = T0 + w[i] * x[i];
      T1 = T1 + wq * x[i];
    }
    float det = S0 * S2 - S1 * S1;
    if (!(det > 0.0f)) break;
    float ns = (S0 * T1 - S1 * T0) / det;
    float nm = (S1 * T1 - S2 * T0) / det;
    if (nm < 0.0f) {
      nm = 0.0f;
      ns = S2 > 0.0f ? T1 / S2 : 0.0f;
    }
    if (ns < 0.0f) {
      ns = 0.0f;
      nm = S0 > 0.0f ? -T0 / S0 : 0.0f;
      if (nm < 0.0f) nm = 0.0f;
    }
    float e = af_err(x, w, n, ns, nm, qmax);
    if (e < be) {
      be = e;
      bs = ns;
      bm = nm;
    }
    s = ns;
    m = nm;
  }
  *s_out = bs;
  *m_out = bm;
}

/*
 * One 84-byte Q2_K block from 256 values x and weights w (layout of the
 * decoder in ds4_oracle.c).  d = max s_j / 15 and dmin = max m_j / 15 rounded
 * to fp16; nibbles sc_j = rint(s_j / d), m_j = rint(m_j / dmin) in 0..15;
 * codes nearest for the stored scale and min.
 */
static void q2k_encode_block(const float* x, const float* w, uint8_t* b) {
  float s[16], m[16];
  float smax = 0.0f, mmax = 0.0f;
  for (int j = 0; j < 16; j++) {
    af_fit(x + 16 * j, w + 16 * j, 16, 3.0f, &s[j], &m[j]);
    smax = fmaxf(smax, s[j]);
    mmax = fmaxf(mmax, m[j]);
  }
  if (!(smax > 0.0f)) smax = 0.0f;  /* +0, whatever zero the maxima kept */
  if (!(mmax > 0.0f)) mmax = 0.0f;
  uint16_t dh = en_f16_bits(smax / 15.0f), mh = en_f16_bits(mmax / 15.0f);
  float d = f16_float(dh), dmin = f16_float(mh);
  memset(b, 0, 84);
  for (int j = 0; j < 16; j++) {
    int sc = d > 0.0f ? (int)clampf(rintf(s[j] / d), 0.0f, 15.0f) : 0;
    int mn = dmin > 0.0f ? (int)clampf(rintf(m[j] / dmin), 0.0f, 15.0f) : 0;
    b[j] = (uint8_t)(sc | (mn << 4));
    float S = d * (float)sc, M = dmin * (float)mn;
    for (int l = 0; l < 16; l++) {
      int i = 16 * j + l;
      int q = q2_code(x[i], S, M);
      int h = i / 128, sh = (i % 128) / 32, c = i % 32;
      b[16 + 32 * h + c] |= (uint8_t)(q << (2 * sh));
    }
  }
  b[80] = (uint8_t)dh;
  b[81] = (uint8_t)(dh >> 8);
  b[82] = (uint8_t)mh;
  b[83] = (uint8_t)(mh >> 8);
}

/* ------------------------------------------------------------------ */
/* Q4_K and Q8_0                                                       */
/* ------------------------------------------------------------------ */

/*
 * One 144-byte Q4_K block (layout of the decoder in ds4_oracle.c) from 256
 * values x and weights w: the Q2_K procedure with 32-value sub-blocks and
 * codes 0..15 (af_fit), d = max s_j / 63 and dmin = max m_j / 63 in fp16,
 * 6-bit nibbles sc_j = rint(s_j / d), m_j = rint(m_j / dmin) in 0..63, codes
 * nearest for the stored pair.
 */
static void q4k_encode_block(const float* x, const float* w, uint8_t* b) {
  float s[8], m[8];
  float smax = 0.0f, mmax = 0.0f;
  for (int j = 0; j < 8; j++) {
    af_fit(x + 32 * j, w + 32 * j, 32, 15.0f, &s[j], &m[j]);
    smax = fmaxf(smax, s[j]);
    mmax = fmaxf(mmax, m[j]);
  }
  if (!(smax > 0.0f)) smax = 0.0f;
  if (!(mmax > 0.0f)) mmax = 0.0f;
  uint16_t dh = en_f16_bits(smax / 63.0f), mh = en_f16_bits(mmax / 63.0f);
  float d = f16_float(dh), dmin = f16_float(mh);
  memset(b, 0, 144);
  b[0] = (uint8_t)dh;
  b[1] = (uint8_t)(dh >> 8);
  b[2] = (uint8_t)mh;
  b[3] = (uint8_t)(mh >> 8);
  uint8_t* S = b + 4;
  for (int j = 0; j < 8; j++) {
    int sc = d > 0.0f ? (int)clampf(rintf(s[j] / d), 0.0f, 63.0f) : 0;
    int mn = dmin > 0.0f ? (int)clampf(rintf(m[j] / dmin), 0.0f, 63.0f) : 0;
    if (j < 4) {
      S[j] = (uint8_t)sc;
      S[j + 4] = (uint8_t)mn;
    } else {
      S[j + 4] = (uint8_t)((sc & 15) | ((mn & 15) << 4));
      S[j - 4] |= (uint8_t)((sc >> 4) << 6);
      S[j] |= (uint8_t)((mn >> 4) << 6);
    }
    float Sc = d * (float)sc, M = dmin * (float)mn;
    for (int l = 0; l < 32; l++) {
      int i = 32 * j + l;
      int q = af_code(x[i], Sc, M, 15.0f);
      int c = i / 64, hi = (i % 64) / 32;
      b[16 + 32 * c + l] |= (uint8_t)(hi ? q << 4 : q);
    }
  }
}

/* One 34-byte Q8_0 block from 32 values: d = max|x| / 127 in fp16, codes
 * rint(x / d) clamped to -127..127 (all zero when d is 0). */
static void q80_encode_block(const float* x, uint8_t* b) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
  uint16_t dh = en_f16_bits(amax / 127.0f);
  float d = f16_float(dh);
  b[0] = (uint8_t)dh;
  b[1] = (uint8_t)(dh >> 8);
  for (int i = 0; i < 32; i++) {
    int q = d > 0.0f ? (int)clampf(rintf(x[i] / d), -127.0f, 127.0f) : 0;
    b[2 + i] = (uint8_t)(int8_t)q;
  }
}

/* ------------------------------------------------------------------ */
/* IQ2_XXS neighbour map                                               */
/* ------------------------------------------------------------------ */

/*
 * Grid values are 8, 25, 43 (levels 0, 1, 2).  A tuple of eight levels has
 * key sum_k level_k 3^k (6561 keys).  Its list: the lowest grid index equal
 * to it when it is on the grid; otherwise every grid entry whose squared
 * level distance is at most the second-smallest distance found over the
 * grid (two shells), in ascending index order.  Layout: count[6561] (u16),
 * then idx[6561][256] (u8).
 */
#define EN_KEYS 6561
#define EN_MAP_BYTES (EN_KEYS * 2 + EN_KEYS * 256)

static int grid_level(uint8_t g) { return g == 8 ? 0 : g == 25 ? 1 : g == 43 ? 2 : -1; }

EXPORT int64_t en_iq2_map_bytes(void) { return EN_MAP_BYTES; }

EXPORT int en_iq2_map_build(const uint8_t* grid, int n_grid, uint8_t* map) {
  if (n_grid < 1 || n_grid > 256) return EN_EINVAL;
  for (int i = 0; i < 8 * n_grid; i++)
    if (grid_level(grid[i]) < 0) return EN_EINVAL;
  uint16_t* count = (uint16_t*)map;
  uint8_t* idx = map + 2 * EN_KEYS;
  for (int key = 0; key < EN_KEYS; key++) {
    int lv[8], k2 = key;
    for (int k = 0; k < 8; k++) {
      lv[k] = k2 % 3;
      k2 /= 3;
    }
    int dist[256];
    int d1 = 1 << 30, d2 = 1 << 30, on = -1;
    for (int i = 0; i < n_grid; i++) {
      int d = 0;
      for (int k = 0; k < 8; k++) {
        int t = lv[k] - grid_level(grid[8 * i + k]);
        d += t * t;
      }
      dist[i] = d;
      if (d == 0 && on < 0) on = i;
      if (d < d1) {
        d2 = d1;
        d1 = d;
      } else if (d > d1 && d < d2) {
        d2 = d;
      }
    }
    int n = 0;
    if (on >= 0) {
      idx[256 * key + n++] = (uint8_t)on;
    } else {
      if (d2 == (1 << 30)) d2 = d1;
      for (int i = 0; i < n_grid; i++)
        if (dist[i] <= d2) idx[256 * key + n++] = (uint8_t)i;
    }
    count[key] = (uint16_t)n;
  }
  return EN_OK;
}

/* ------------------------------------------------------------------ */
/* IQ2_XXS                                                             */
/* ------------------------------------------------------------------ */

static int iq2_level(float v) { return v < 16.5f ? 0 : v < 34.0f ? 1 : 2; }

/* Grid index of the 8 targets t (weights w) at group scale S > 0: the
 * nearest level of each t/S (thresholds half-way between 8, 25, 43), then
 * the key's list; among several entries the lowest weighted squared error
 * sum_k w_k (t_k - S g_k)^2, first in list order on ties. */
static int iq2_pick(const float* t, const float* w, float S, const uint8_t* grid,
                    const uint8_t* map) {
  int key = 0, p = 1;
  for (int k = 0; k < 8; k++) {
    key += iq2_level(t[k] / S) * p;
    p *= 3;
  }
  const uint16_t* count = (const uint16_t*)map;
  const uint8_t* list = map + 2 * EN_KEYS + 256 * key;
  int n = count[key], best = list[0];
  if (n == 1) return best;
  float be = INFINITY;
  for (int j = 0; j < n; j++) {
    int i = list[j];
    float e = 0.0f;
    for (int k = 0; k < 8; k++) {
      float r = S * (float)grid[8 * i + k];
      r = t[k] - r;
      e = e + w[k] * (r * r);
    }
    if (e < be) {
      be = e;
      best = i;
    }
  }
  return best;
}

/*
 * One 66-byte IQ2_XXS block (layout of the decoder in ds4_oracle.c) from 256
 * values x and weights w.  Per group of 32 values:
 *   signs: sigma_k = -1 where x_k < 0; in a tuple of 8 with an odd number of
 *     negatives, the sign of the value with the smallest w_k x_k^2 (lowest k
 *     on ties) is flipped, since the format stores an even number; targets
 *     t_k = sigma_k x_k.
 *   scale: with tmax = max t_k (a group with tmax <= 0 keeps scale 0), 16
 *     candidates S_c = tmax / (24 + 2c), c = 0..15; each assigns the four
 *     tuples (iq2_pick), refits S = sum w t g / sum w g^2 for them (kept when
 *     both sums are positive) and is scored by sum w (t - S g)^2 over the 32
 *     values; the lowest score wins, the first candidate on ties.
 * Block: d = 8 max S_g / 31 rounded to fp16; nibble s_g = rint((8 S_g / d -
 * 1) / 2) in 0..15; the tuples are assigned again at the stored scale
 * d (2 s_g + 1) / 8 (when that is 0, every tuple takes the first entry of the
 * all-zero-level key).
 */
static void iq2_encode_block(const float* x, const float* w, const uint8_t* grid,
                             const uint8_t* map, uint8_t* b) {
  float t[256], Sg[8];
  uint32_t signs[8];
  for (int g = 0; g < 8; g++) {
    signs[g] = 0;
    for (int u = 0; u < 4; u++) {
      const int o = 32 * g + 8 * u;
      int neg = 0, n = 0;
      for (int k = 0; k < 8; k++)
        if (x[o + k] < 0.0f) {
          neg |= 1 << k;
          n++;
        }
      if (n & 1) {
        int kmin = 0;
        float emin = w[o] * (x[o] * x[o]);
        for (int k = 1; k < 8; k++) {
          float e = w[o + k] * (x[o + k] * x[o + k]);
          if (e < emin) {
            emin = e;
            kmin = k;
          }
        }
        neg ^= 1 << kmin;
      }
      for (int k = 0; k < 8; k++) t[o + k] = ((neg >> k) & 1) ? -x[o + k] : x[o + k];
      signs[g] |= (uint32_t)(neg & 0x7F) << (7 * u);
    }
    const float* tg = t + 32 * g;
    const float* wg = w + 32 * g;
    float tmax = tg[0];
    for (int k = 1; k < 32; k++) tmax = fmaxf(tmax, tg[k]);
    Sg[g] = 0.0f;
    if (!(tmax > 0.0f)) continue;
    float be = INFINITY;
    for (int c = 0; c < 16; c++) {
      float S = tmax / (float)(24 + 2 * c);
      int id[4];
      for (int u = 0; u < 4; u++) id[u] = iq2_pick(tg + 8 * u, wg + 8 * u, S, grid, map);
      float num = 0.0f, den = 0.0f;
      for (int k = 0; k < 32; k++) {
        float gv = (float)grid[8 * id[k / 8] + k % 8];
        num = num + (wg[k] * tg[k]) * gv;
        den = den + (wg[k] * gv) * gv;
      }
      if (num > 0.0f && den > 0.0f) S = num / den;
      float e = 0.0f;
      for (int k = 0; k < 32; k++) {
        float r = S * (float)grid[8 * id[k / 8] + k % 8];
        r = tg[k] - r;
        e = e + wg[k] * (r * r);
      }
      if (e < be) {
        be = e;
        Sg[g] = S;
      }
    }
  }
  float smax = 0.0f;
  for (int g = 0; g < 8; g++) smax = fmaxf(smax, Sg[g]);
  if (!(smax > 0.0f)) smax = 0.0f;
  uint16_t dh = en_f16_bits((smax * 8.0f) / 31.0f);
  float d = f16_float(dh);
  b[0] = (uint8_t)dh;
  b[1] = (uint8_t)(dh >> 8);
  for (int g = 0; g < 8; g++) {
    int s = d > 0.0f ? (int)clampf(rintf(((Sg[g] * 8.0f) / d - 1.0f) / 2.0f), 0.0f, 15.0f) : 0;
    float S = (d * (float)(2 * s + 1)) / 8.0f;
    uint8_t* gp = b + 2 + 8 * g;
    for (int u = 0; u < 4; u++) {
      int id;
      if (S > 0.0f) {
        id = iq2_pick(t + 32 * g + 8 * u, w + 32 * g + 8 * u, S, grid, map);
      } else {
        id = map[2 * EN_KEYS];  /* first entry of key 0 */
      }
      gp[u] = (uint8_t)id;
    }
    uint32_t word = signs[g] | ((uint32_t)s << 28);
    for (int k = 0; k < 4; k++) gp[4 + k] = (uint8_t)(word >> (8 * k));
  }
}

/* ------------------------------------------------------------------ */
/* Matrices                                                            */
/* ------------------------------------------------------------------ */

/*
 * Encode n_mats matrices [rows][cols] of src (row-major, stacked) into blocks
 * tiling each row (cols % 256 == 0).  importance: NULL (every weight 1; Q2_K,
 * Q4_K and Q8_0, which uses none) or n_mats vectors of cols values, matrix m's at importance +
 * m * imp_stride (0: one vector for all); the weight of a value is its
 * column's importance.  IQ2_XXS needs the grid (256 x 8 bytes of 8, 25, 43)
 * and its map (en_iq2_map_build).  Values must be finite and weights finite
 * and >= 0 (else EN_EINVAL, nothing written).
 */
EXPORT int en_quantize(int qt, const float* src, int64_t n_mats, int64_t rows, int64_t cols,
                       const float* importance, int64_t imp_stride, const uint8_t* grid,
                       const uint8_t* map, uint8_t* dst) {
  if (qt < EN_Q2_K || qt > EN_Q4_K || n_mats < 0 || rows < 0 || cols < 0 || cols % 256 != 0 ||
      imp_stride < 0)
    return EN_EINVAL;
  if (qt == EN_IQ2_XXS && (!importance || !grid || !map)) return EN_EINVAL;
  int64_t n = n_mats * rows * cols;
  for (int64_t i = 0; i < n; i++)
    if (!isfinite(src[i])) return EN_EINVAL;
  if (importance) {
    int64_t n_vec = imp_stride ? n_mats : 1;
    for (int64_t v = 0; v < n_vec; v++)
      for (int64_t c = 0; c < cols; c++) {
        float x = importance[v * imp_stride + c];
        if (!isfinite(x) || x < 0.0f) return EN_EINVAL;
      }
  }
  const int bb = qt == EN_Q2_K ? 84 : qt == EN_IQ2_XXS ? 66 : qt == EN_Q4_K ? 144 : 8 * 34;
  const int64_t bpr = cols / 256;
  float unit[256];
  for (int i = 0; i < 256; i++) unit[i] = 1.0f;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_mats * rows; r++) {
    const int64_t m = r / (rows ? rows : 1);
    const float* imp = importance ? importance + m * imp_stride : NULL;
    for (int64_t blk = 0; blk < bpr; blk++) {
      const float* x = src + r * cols + 256 * blk;
      const float* w = imp ? imp + 256 * blk : unit;
      uint8_t* b = dst + (r * bpr + blk) * bb;
      if (qt == EN_Q2_K) q2k_encode_block(x, w, b);
      else if (qt == EN_Q4_K) q4k_encode_block(x, w, b);
      else if (qt == EN_Q8_0)
        for (int g = 0; g < 8; g++) q80_encode_block(x + 32 * g, b + 34 * g);  /* 8 blocks per 256 */
      else iq2_encode_block(x, w, grid, map, b);
    }
  }
  return EN_OK;
}

/* Fallback importance (DS4C2 sec. 8): the column energy sum_r W[r][c]^2 of
 * each of n_mats matrices [rows][cols], in fp64, out[m][c]. */
EXPORT void en_column_energy(const float* src, int64_t n_mats, int64_t rows, int64_t cols,
                             double* out) {
  for (int64_t m = 0; m < n_mats; m++)
    for (int64_t c = 0; c < cols; c++) {
      double e = 0.0;
      for (int64_t r = 0; r < rows; r++) {
        double v = (double)src[(m * rows + r) * cols + c];
        e += v * v;
      }
      out[m * cols + c] = e;
    }
}
