/*
 * ds4_oracle.c -- plain, slow CPU reference of the routed-expert MoE FFN on
 * 2-bit block-quantised weights.  TEST INFRASTRUCTURE ONLY: the test suite,
 * the smoke check and the benchmark's CPU-baseline leg call it; the GPU
 * library never does, and the two share no code.
 *
 * Everything is evaluated in fp64 (router logits exactly, sqrtsoftplus in
 * binary128) and rounded once at the end of each step to the storage type
 * the step's result is defined in.  No blocking, fusion or reordering beyond
 * what the definitions below state.  Rows may be computed by several OpenMP
 * threads; each row's sum runs sequentially, so results do not depend on
 * the thread count.
 *
 * Pages cited (the method is defined there; formats partly by reading):
 *   FLOW  = qiita.com/sukimaengineer/items/cd76fec76d49a098abed
 *           (DeepSeek-V4-Flash config numbers and one-token compute flow)
 *   DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec
 *           ("[#2] ds4.c を読み解く": asymmetric 2-bit quantisation)
 * Where the pages leave a step open, the reading taken is stated at the
 * function.  The IQ2_XXS group-scale mapping (2s+1)/8 is such a reading:
 * parity unpinned by the pages (pinned only by its own written definition).
 *
 * Build: gcc -O2 -fPIC -shared -std=gnu11 -fopenmp -ffp-contract=off
 *        -o liboracle.so ds4_oracle.c -lquadmath -lm
 */
#define _GNU_SOURCE
#include <math.h>
#include <quadmath.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_Q2_K = 0, OR_IQ2_XXS = 1, OR_Q8_0 = 2, OR_Q4_K = 3 };
enum { OR_OK = 0, OR_EINVAL = -1, OR_EUNCERTAIN = -6 };

/* ------------------------------------------------------------------ */
/* Scalar formats                                                      */
/* ------------------------------------------------------------------ */

/* IEEE binary16 bit pattern -> exact double. */
EXPORT double or_f16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* bfloat16 bit pattern -> exact double (the top half of a binary32). */
EXPORT double or_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double load_elem(const void* p, int dt, int64_t i) {
  if (dt == OR_F32) return (double)((const float*)p)[i];
  if (dt == OR_F16) return or_f16_value(((const uint16_t*)p)[i]);
  return or_bf16_value(((const uint16_t*)p)[i]);
}

/* Round a finite double to the nearest bfloat16 (ties to even); returns bits. */
EXPORT uint16_t or_round_bf16(double v) {
  if (v == 0.0 || isnan(v) || isinf(v)) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
  }
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
  /* bfloat16 keeps 8 significant bits; below 2^-126 the quantum is 2^-133. */
  int q_exp = e - 8;
  if (q_exp < -133) q_exp = -133;
  double r = ldexp(rint(ldexp(v, -q_exp)), q_exp); /* rint: ties to even */
  /* rounding past the largest finite bfloat16 (0x1.FEp127) gives infinity */
  float f = fabs(r) > 0x1.FEp127 ? (r > 0 ? INFINITY : -INFINITY) : (float)r;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Block decoders (DS4C2 sec. 3 and 4; FLOW sec. on Dwarf Star quant)  */
/* ------------------------------------------------------------------ */

static uint32_t rd_u32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint16_t rd_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/*
 * Q2_K, 84 bytes per 256 values (DS4C2 sec. 3, layout table and packing):
 *   bytes  0..15  one byte per 16-value sub-block j: low nibble = scale sc_j,
 *                 high nibble = min m_j (nibble order: reading)
 *   bytes 16..79  2-bit codes; byte 32h+l holds the codes of values
 *                 128h+l, +32, +64, +96 in bit pairs 0-1, 2-3, 4-5, 6-7
 *   bytes 80..81  fp16 d (scale base), 82..83 fp16 dmin (min base), LE
 *   value i:  y = d * sc_j * q_i - dmin * m_j,   j = i / 16
 * The min is subtracted (the affine "d*q + m" of FLOW is written loosely).
 */
static void decode_q2k(const uint8_t* b, double* y) {
  double d = or_f16_value(rd_u16(b + 80)), dmin = or_f16_value(rd_u16(b + 82));
  for (int i = 0; i < 256; i++) {
    int h = i / 128, s = (i % 128) / 32, l = i % 32, j = i / 16;
    int q = (b[16 + 32 * h + l] >> (2 * s)) & 3;
    int sc = b[j] & 0xF, m = b[j] >> 4;
    y[i] = d * (double)sc * (double)q - dmin * (double)m;
  }
}

/*
 * IQ2_XXS-style, 66 bytes per 256 values (DS4C2 sec. 4: eight 32-value
 * groups, four 8-value grid indices and four 7-bit sign masks per group,
 * fp16 block scale refined by a 4-bit group nibble, 256-entry grid):
 *   bytes 0..1      fp16 d
 *   group g (0..7)  bytes 2+8g .. 9+8g: idx_k = byte k (k=0..3), then a LE
 *                   u32 w: sign7_k = (w >> 7k) & 0x7F, s = w >> 28
 *   sign8_k = sign7_k with bit 7 set when popcount(sign7_k) is odd
 *   value 32g+8k+j = d * (2s+1)/8 * grid[idx_k][j] * (bit j of sign8_k ? -1 : +1)
 * Readings: byte order inside a group, the even-parity eighth sign, a set
 * bit meaning negative, and the (2s+1)/8 refinement of d.
 */
static void decode_iq2xxs(const uint8_t* b, const uint8_t* grid, double* y) {
  double d = or_f16_value(rd_u16(b));
  for (int g = 0; g < 8; g++) {
    const uint8_t* gp = b + 2 + 8 * g;
    uint32_t w = rd_u32(gp + 4);
    int s = (int)(w >> 28);
    double dg = d * (double)(2 * s + 1) / 8.0;
    for (int k = 0; k < 4; k++) {
      int idx = gp[k];
      int sign7 = (int)((w >> (7 * k)) & 0x7F);
      int par = __builtin_popcount((unsigned)sign7) & 1;
      int sign8 = sign7 | (par << 7);
      for (int j = 0; j < 8; j++) {
        double v = dg * (double)grid[idx * 8 + j];
        y[32 * g + 8 * k + j] = ((sign8 >> j) & 1) ? -v : v;
      }
    }
  }
}

/* Q8_0, 34 bytes per 32 values: fp16 d, then 32 int8 codes; y = d * c
 * (FLOW sec. on Dwarf Star quant: symmetric, one scale per 32 values). */
static void decode_q80(const uint8_t* b, double* y) {
  double d = or_f16_value(rd_u16(b));
  for (int i = 0; i < 32; i++) y[i] = d * (double)(int8_t)b[2 + i];
}

/*
 * Q4_K, 144 bytes per 256 values.  The pages give the size (DS4C2 sec. 3,
 * type table: q4_K, 256 values, 144 bytes), say that Q2_K and Q4_K are
 * affine formats with a scale and a minimum per sub-block of a super-block
 * (FLOW, quantisation section), and leave the layout to the ggml k-quant
 * family.  Reading (that family's layout; 2 + 2 + 12 + 128 = 144 bytes):
 *   bytes 0..1 fp16 d, 2..3 fp16 dmin (LE)
 *   bytes 4..15 six-bit scale sc_j and min m_j of the 32-value sub-blocks
 *     j = 0..7:  j < 4:  sc_j = S[j] & 63,  m_j = S[j+4] & 63
 *                j >= 4: sc_j = (S[j+4] & 15) | (S[j-4] >> 6) << 4
 *                        m_j  = (S[j+4] >> 4) | (S[j] >> 6) << 4   (S = bytes 4..15)
 *   bytes 16..143 four-bit codes: byte 16+32c+l holds value 64c+l in its
 *     low nibble and value 64c+32+l in its high nibble (c < 4, l < 32)
 *   value i:  y = d * sc_j * q_i - dmin * m_j,   j = i / 32
 */
static void decode_q4k(const uint8_t* b, double* y) {
  double d = or_f16_value(rd_u16(b)), dmin = or_f16_value(rd_u16(b + 2));
  const uint8_t* S = b + 4;
  for (int i = 0; i < 256; i++) {
    int c = i / 64, l = i % 32, hi = (i % 64) / 32, j = i / 32;
    int byte = b[16 + 32 * c + l];
    int q = hi ? byte >> 4 : byte & 15;
    int sc, m;
    if (j < 4) {
      sc = S[j] & 63;
      m = S[j + 4] & 63;
    } else {
      sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
      m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
    y[i] = d * (double)sc * (double)q - dmin * (double)m;
  }
}

static int block_bytes(int qt) {
  return qt == OR_Q2_K ? 84 : qt == OR_IQ2_XXS ? 66 : qt == OR_Q4_K ? 144 : 34;
}
static int block_vals(int qt) { return qt == OR_Q8_0 ? 32 : 256; }

/* Decode n consecutive blocks (the row-major flattening of a matrix). */
EXPORT int or_dequant(int qt, const uint8_t* blocks, int64_t n_blocks, const uint8_t* grid,
                      double* out) {
  if (qt < 0 || qt > 3 || (qt == OR_IQ2_XXS && !grid)) return OR_EINVAL;
  int bb = block_bytes(qt), bv = block_vals(qt);
  /* blocks are independent: threads split them, results do not change */
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_blocks; i++) {
    const uint8_t* b = blocks + i * bb;
    double* y = out + i * bv;
    if (qt == OR_Q2_K) decode_q2k(b, y);
    else if (qt == OR_IQ2_XXS) decode_iq2xxs(b, grid, y);
    else if (qt == OR_Q4_K) decode_q4k(b, y);
    else decode_q80(b, y);
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Exact dot product rounded once to binary32                          */
/* ------------------------------------------------------------------ */

/* Fixed-point accumulator: bit k of the magnitude has weight 2^(k - LOW). */
#define ACC_LOW 1120
#define ACC_LIMBS 72 /* 32-bit payload per limb: bits 0 .. 2303 */

typedef struct {
  uint64_t pos[ACC_LIMBS];
  uint64_t neg[ACC_LIMBS];
} exact_acc;

static void acc_add(exact_acc* a, double v) {
  if (v == 0.0) return;
  int e;
  double m = frexp(fabs(v), &e);            /* |v| = m 2^e */
  uint64_t mi = (uint64_t)ldexp(m, 53);      /* exact 53-bit integer */
  int pos = e - 53 + ACC_LOW;                /* weight of mi's bit 0 */
  if (pos < 0 || pos + 53 >= ACC_LIMBS * 32 - 40) abort();
  uint64_t* L = v < 0 ? a->neg : a->pos;
  int limb = pos / 32, sh = pos % 32;
  unsigned __int128 s = (unsigned __int128)mi << sh; /* at most 85 bits */
  L[limb] += (uint64_t)(s & 0xFFFFFFFFu);
  L[limb + 1] += (uint64_t)((s >> 32) & 0xFFFFFFFFu);
  L[limb + 2] += (uint64_t)(s >> 64);
}

static void acc_normalize(uint64_t* L) {
  uint64_t carry = 0;
  for (int i = 0; i < ACC_LIMBS; i++) {
    uint64_t t = L[i] + carry;
    L[i] = t & 0xFFFFFFFFULL;
    carry = t >> 32;
  }
  if (carry) abort();
}

/* Round the signed accumulator value to the nearest binary32, ties to even. */
static float acc_to_f32(exact_acc* a) {
  acc_normalize(a->pos);
  acc_normalize(a->neg);
  int cmp = 0;
  for (int i = ACC_LIMBS - 1; i >= 0 && !cmp; i--)
    cmp = a->pos[i] > a->neg[i] ? 1 : a->pos[i] < a->neg[i] ? -1 : 0;
  if (cmp == 0) return 0.0f;
  uint64_t* big = cmp > 0 ? a->pos : a->neg;
  uint64_t* small = cmp > 0 ? a->neg : a->pos;
  uint32_t D[ACC_LIMBS];
  int64_t borrow = 0;
  for (int i = 0; i < ACC_LIMBS; i++) {
    int64_t t = (int64_t)big[i] - (int64_t)small[i] - borrow;
    borrow = t < 0;
    D[i] = (uint32_t)(t + (borrow ? (1LL << 32) : 0));
  }
  int top = -1;
  for (int i = ACC_LIMBS - 1; i >= 0 && top < 0; i--)
    if (D[i]) top = i * 32 + 31 - __builtin_clz(D[i]);
#define BIT(k) ((k) >= 0 ? (int)((D[(k) / 32] >> ((k) % 32)) & 1u) : 0)
  int cut = top - 23;                          /* keep 24 significant bits */
  int sub_cut = -149 + ACC_LOW;                /* binary32 subnormal quantum */
  if (cut < sub_cut) cut = sub_cut;
  uint64_t M = 0;
  for (int k = top; k >= cut; k--) M = (M << 1) | (uint64_t)BIT(k);
  int guard = BIT(cut - 1);
  int sticky = 0;
  for (int k = cut - 2; k >= 0 && !sticky; k--) sticky = BIT(k);
#undef BIT
  if (guard && (sticky || (M & 1))) M++;
  double r = ldexp((double)M, cut - ACC_LOW);  /* exact in double */
  float f = (float)r;                           /* exact, or overflow to inf */
  return cmp > 0 ? f : -f;
}

/* RN_f32( exact sum_i x_i * w_i ).  Each product of two binary16/bfloat16/
 * binary32 values is exact in binary64; the sum is then accumulated
 * exactly, so the result does not depend on any summation order. */
EXPORT float or_exact_dot(const void* x, int xdt, const void* w, int wdt, int64_t n) {
  exact_acc* a = (exact_acc*)calloc(1, sizeof(exact_acc));
  for (int64_t i = 0; i < n; i++) {
    double xi = load_elem(x, xdt, i), wi = load_elem(w, wdt, i);
    double p = xi * wi;
    if (fma(xi, wi, -p) != 0.0) abort(); /* product must be exact */
    acc_add(a, p);
  }
  float r = acc_to_f32(a);
  free(a);
  return r;
}

/* ------------------------------------------------------------------ */
/* Router (FLOW, config table and "MoE FFN" section)                   */
/* ------------------------------------------------------------------ */

/*
 * sqrtsoftplus: s = sqrt(softplus(z)) = sqrt(ln(1 + e^z)), the plain reading
 * of the scoring name; correctly rounded to binary32.  Evaluated in binary128
 * (softplus written as max(z,0) + ln(1 + e^-|z|) so e^z never overflows).  The
 * result is accepted only if a 2^-100 relative perturbation cannot change the
 * binary32 rounding; otherwise the oracle aborts loudly.
 */
EXPORT float or_sqrtsoftplus(float zf) {
  __float128 z = (__float128)zf;
  __float128 az = z < 0 ? -z : z;
  __float128 sp = (z > 0 ? z : (__float128)0) + log1pq(expq(-az));
  __float128 s = sqrtq(sp);
  float r = (float)s;
  __float128 eps = s * 0x1p-100Q;
  if ((float)(s - eps) != r || (float)(s + eps) != r) abort();
  return r;
}

static int key_before(float ka, int a, float kb, int b) {
  return ka > kb || (ka == kb && a < b);
}

/*
 * Routed layer, per token (FLOW "MoE FFN" section):
 *   z_e   = RN_f32(exact x . W[e])              W stored [E][H], one row per expert
 *   s_e   = sqrtsoftplus(z_e)
 *   key_e = RN_f32(s_e + b_e)                    bias used for selection only (noaux_tc)
 *   ids   = the K largest keys, ties to the lower expert index, slots ordered
 *           by key descending then index ascending (flat top-K, no groups)
 *   w_k   = RN_f32(scale * s_k / sum_j s_j)      sum in fp64, slot order
 * (norm_topk_prob, then routed_scaling_factor = scale = 1.5).
 */
EXPORT int or_route(int T, int H, int E, int K, const void* x, int xdt, const void* W, int wdt,
                    const float* bias, double scale, int32_t* ids, float* wts, float* logits,
                    float* scores) {
  if (T < 0 || H <= 0 || E <= 0 || K <= 0 || K > E) return OR_EINVAL;
  int esz = wdt == OR_F32 ? 4 : 2, xsz = xdt == OR_F32 ? 4 : 2;
  float* z = (float*)malloc(sizeof(float) * E);
  float* s = (float*)malloc(sizeof(float) * E);
  float* key = (float*)malloc(sizeof(float) * E);
  char* taken = (char*)malloc(E);
  for (int t = 0; t < T; t++) {
    const char* xt = (const char*)x + (int64_t)t * H * xsz;
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; e++) {
      z[e] = or_exact_dot(xt, xdt, (const char*)W + (int64_t)e * H * esz, wdt, H);
      s[e] = or_sqrtsoftplus(z[e]);
      key[e] = s[e] + bias[e];
    }
    memset(taken, 0, E);
    for (int k = 0; k < K; k++) {
      int best = -1;
      for (int e = 0; e < E; e++)
        if (!taken[e] && (best < 0 || key_before(key[e], e, key[best], best))) best = e;
      taken[best] = 1;
      ids[t * K + k] = best;
    }
    double sum = 0.0;
    for (int k = 0; k < K; k++) sum += (double)s[ids[t * K + k]];
    for (int k = 0; k < K; k++) wts[t * K + k] = (float)(scale * (double)s[ids[t * K + k]] / sum);
    if (logits) memcpy(logits + (int64_t)t * E, z, sizeof(float) * E);
    if (scores) memcpy(scores + (int64_t)t * E, s, sizeof(float) * E);
  }
  free(z);
  free(s);
  free(key);
  free(taken);
  return OR_OK;
}

/*
 * Hash-routed layer (FLOW: the first three layers have no router; expert ids
 * come from the static token-id table tid2eid).  ids = table[token][0..K-1]
 * in table order; gate weights are equal, scale/K each (reading: keeps the
 * routed sum at the scaling factor).  Returns OR_EINVAL on a token id out of
 * range or a table row with an id out of range or repeated.
 */
EXPORT int or_route_hash(int T, int K, int E, const int32_t* tok, const int32_t* table, int vocab,
                         double scale, int32_t* ids, float* wts) {
  for (int t = 0; t < T; t++) {
    if (tok[t] < 0 || tok[t] >= vocab) return OR_EINVAL;
    const int32_t* row = table + (int64_t)tok[t] * K;
    for (int k = 0; k < K; k++) {
      if (row[k] < 0 || row[k] >= E) return OR_EINVAL;
      for (int q = 0; q < k; q++)
        if (row[q] == row[k]) return OR_EINVAL;
      ids[t * K + k] = row[k];
      wts[t * K + k] = (float)(scale / (double)K);
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Token -> expert permutation                                         */
/* ------------------------------------------------------------------ */

static int cmp_pairs(const void* pa, const void* pb, void* ctx) {
  const int32_t* ids = (const int32_t*)ctx;
  int a = *(const int*)pa, b = *(const int*)pb;
  int ea = ids[a], eb = ids[b];
  if (ea != eb) return ea < eb ? -1 : 1;
  return a < b ? -1 : (a > b);
}

/*
 * Pair p = t*K + k (token t, slot k).  Pairs are ordered by the key
 * (expert, t, k); counts[e] = pairs routed to e; offsets = exclusive prefix
 * sum of counts (E+1 entries); perm[i] = pair at sorted position i;
 * inv[p] = position of pair p.  Returns OR_EINVAL for an id outside [0,E).
 */
EXPORT int or_permute(int T, int K, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                      int32_t* perm, int32_t* inv) {
  int n = T * K;
  for (int p = 0; p < n; p++)
    if (ids[p] < 0 || ids[p] >= E) return OR_EINVAL;
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (int p = 0; p < n; p++) counts[ids[p]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  for (int p = 0; p < n; p++) perm[p] = p;
  qsort_r(perm, (size_t)n, sizeof(int32_t), cmp_pairs, (void*)ids);
  for (int i = 0; i < n; i++) inv[perm[i]] = i;
  return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Expert FFN and weighted combine (FLOW "MoE FFN" section)            */
/* ------------------------------------------------------------------ */

/* y[r] = sum_c A[r][c] * v[c], fp64, each row summed in column order. */
static void matvec(const double* A, const double* v, int64_t R, int64_t C, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; r++) {
    double acc = 0.0;
    const double* a = A + r * C;
    for (int64_t c = 0; c < C; c++) acc += a[c] * v[c];
    y[r] = acc;
  }
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* E(x) = W_down (SiLU(W_gate x) * (W_up x)), all in fp64 on decoded weights. */
static void swiglu_expert(const double* Wg, const double* Wu, const double* Wd, const double* x,
                          int64_t H, int64_t I, double* g, double* u, double* y) {
  matvec(Wg, x, I, H, g);
  matvec(Wu, x, I, H, u);
  for (int64_t i = 0; i < I; i++) g[i] = silu(g[i]) * u[i];
  matvec(Wd, g, H, I, y);
}

static double* decode_matrix(int qt, const uint8_t* data, int64_t R, int64_t C, const uint8_t* grid) {
  int64_t nv = R * C;
  double* m = (double*)malloc(sizeof(double) * nv);
  if (!m) abort();
  or_dequant(qt, data, nv / block_vals(qt), grid, m);
  return m;
}

/*
 * out_t = sum_k w_tk * E_{ids[t][k]}(x_t)  (+ shared(x_t), not scaled)
 * for the tokens listed in `tokens` (n_tok of them, indices into x/ids/wts),
 * written to out[n_tok][H] as RN_f32 of the fp64 result.
 *
 * Expert matrices: gate/up are [I][H], down is [H][I], each the row-major
 * flattening of a stacked tensor tiled by blocks (FLOW / DS4C2: all experts
 * of a layer in one tensor).  expert_gate[e] etc. point at expert e's bytes
 * (NULL for experts not supplied; using one is an error).  The shared expert
 * (nullable) has intermediate size sh_I.  routed_scale is already folded into
 * the weights wts (they sum to it), so no further factor is applied here.
 */
EXPORT int or_moe_ffn(int H, int I, int E, int K, const void* x, int xdt, const int32_t* ids,
                      const float* wts, const int32_t* tokens, int n_tok, int gate_qt,
                      const uint8_t* const* expert_gate, int up_qt, const uint8_t* const* expert_up,
                      int down_qt, const uint8_t* const* expert_down, const uint8_t* grid, int sh_I,
                      int sh_qt, const uint8_t* sh_gate, const uint8_t* sh_up,
                      const uint8_t* sh_down, float* out) {
  if (H <= 0 || I <= 0 || E <= 0 || K <= 0 || n_tok < 0) return OR_EINVAL;
  int xsz = xdt == OR_F32 ? 4 : 2;
  double* acc = (double*)calloc((size_t)n_tok * H, sizeof(double));
  double* xv = (double*)malloc(sizeof(double) * (size_t)n_tok * H);
  for (int i = 0; i < n_tok; i++)
    for (int c = 0; c < H; c++)
      xv[(int64_t)i * H + c] = load_elem((const char*)x + (int64_t)tokens[i] * H * xsz, xdt, c);
  int64_t Imax = I > sh_I ? I : sh_I;
  double* g = (double*)malloc(sizeof(double) * Imax);
  double* u = (double*)malloc(sizeof(double) * Imax);
  double* y = (double*)malloc(sizeof(double) * H);
  int rc = OR_OK;
  for (int e = 0; e < E && rc == OR_OK; e++) {
    int used = 0;
    for (int i = 0; i < n_tok; i++)
      for (int k = 0; k < K; k++) used |= ids[tokens[i] * K + k] == e;
    if (!used) continue;
    if (!expert_gate[e] || !expert_up[e] || !expert_down[e]) { rc = OR_EINVAL; break; }
    double* Wg = decode_matrix(gate_qt, expert_gate[e], I, H, grid);
    double* Wu = decode_matrix(up_qt, expert_up[e], I, H, grid);
    double* Wd = decode_matrix(down_qt, expert_down[e], H, I, grid);
    for (int i = 0; i < n_tok; i++)
      for (int k = 0; k < K; k++) {
        if (ids[tokens[i] * K + k] != e) continue;
        swiglu_expert(Wg, Wu, Wd, xv + (int64_t)i * H, H, I, g, u, y);
        double w = (double)wts[tokens[i] * K + k];
        for (int c = 0; c < H; c++) acc[(int64_t)i * H + c] += w * y[c];
      }
    free(Wg);
    free(Wu);
    free(Wd);
  }
  if (rc == OR_OK && sh_gate) {
    double* Wg = decode_matrix(sh_qt, sh_gate, sh_I, H, grid);
    double* Wu = decode_matrix(sh_qt, sh_up, sh_I, H, grid);
    double* Wd = decode_matrix(sh_qt, sh_down, H, sh_I, grid);
    for (int i = 0; i < n_tok; i++) {
      swiglu_expert(Wg, Wu, Wd, xv + (int64_t)i * H, H, sh_I, g, u, y);
      for (int c = 0; c < H; c++) acc[(int64_t)i * H + c] += y[c];
    }
    free(Wg);
    free(Wu);
    free(Wd);
  }
  if (rc == OR_OK)
    for (int64_t j = 0; j < (int64_t)n_tok * H; j++) out[j] = (float)acc[j];
  free(acc);
  free(xv);
  free(g);
  free(u);
  free(y);
  return rc;
}

/* ------------------------------------------------------------------ */
/* Importance statistics of the routed experts' inputs (DS4C2 sec. 5,  */
/* "imatrix": activation statistics, not weight statistics; sec. 7:    */
/* one entry of n_expert * n_columns values per tensor)                */
/* ------------------------------------------------------------------ */

/*
 * For every token t < T and slot k < K with e = ids[t][k]:
 *   gu[e][c] += x[t][c]^2                 (c < H: the gate/up input, i.e. the
 *                                          FFN-normalised activation as given)
 *   dn[e][i] += (w_tk * h_tk[i])^2        (i < I: the down input, the SwiGLU
 *                                          row of the pair after its routing
 *                                          weight is applied)
 * with h_tk = SiLU(W_gate[e] x_t) * (W_up[e] x_t) in fp64.  Reading: the
 * routing weight is the one the layer multiplies the expert's output by (it
 * includes the routed scaling, so the weights of a token sum to 1.5).  gu and
 * dn (E*H and E*I doubles) are accumulated into, in token-then-slot order.
 */
EXPORT int or_imatrix(int H, int I, int E, int K, int T, const void* x, int xdt,
                      const int32_t* ids, const float* wts, int gate_qt,
                      const uint8_t* const* expert_gate, int up_qt,
                      const uint8_t* const* expert_up, const uint8_t* grid, double* gu,
                      double* dn) {
  if (H <= 0 || I <= 0 || E <= 0 || K <= 0 || T < 0) return OR_EINVAL;
  int xsz = xdt == OR_F32 ? 4 : 2;
  for (int64_t j = 0; j < (int64_t)T * K; j++)
    if (ids[j] < 0 || ids[j] >= E) return OR_EINVAL;
  double* xv = (double*)malloc(sizeof(double) * H);
  double* g = (double*)malloc(sizeof(double) * I);
  double* u = (double*)malloc(sizeof(double) * I);
  int rc = OR_OK;
  for (int e = 0; e < E && rc == OR_OK; e++) {
    int used = 0;
    for (int64_t j = 0; j < (int64_t)T * K; j++) used |= ids[j] == e;
    if (!used) continue;
    if (!expert_gate[e] || !expert_up[e]) { rc = OR_EINVAL; break; }
    double* Wg = decode_matrix(gate_qt, expert_gate[e], I, H, grid);
    double* Wu = decode_matrix(up_qt, expert_up[e], I, H, grid);
    for (int t = 0; t < T; t++)
      for (int k = 0; k < K; k++) {
        if (ids[(int64_t)t * K + k] != e) continue;
        for (int c = 0; c < H; c++) {
          xv[c] = load_elem((const char*)x + (int64_t)t * H * xsz, xdt, c);
          gu[(int64_t)e * H + c] += xv[c] * xv[c];
        }
        matvec(Wg, xv, I, H, g);
        matvec(Wu, xv, I, H, u);
        double w = (double)wts[(int64_t)t * K + k];
        for (int i = 0; i < I; i++) {
          double v = w * (silu(g[i]) * u[i]);
          dn[(int64_t)e * I + i] += v * v;
        }
      }
    free(Wg);
    free(Wu);
  }
  free(xv);
  free(g);
  free(u);
  return rc;
}

/* ------------------------------------------------------------------ */
/* RMSNorm before the MoE block, residual add after (FLOW token flow)  */
/* ------------------------------------------------------------------ */

/* xn[t][c] = RN_bf16( h[t][c] * (mean_c h^2 + eps)^(-1/2) * w[c] ), fp64. */
EXPORT int or_rmsnorm_bf16(int T, int H, const float* h, const float* w, double eps,
                           uint16_t* xn) {
  for (int t = 0; t < T; t++) {
    const float* ht = h + (int64_t)t * H;
    double ss = 0.0;
    for (int c = 0; c < H; c++) ss += (double)ht[c] * (double)ht[c];
    double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int c = 0; c < H; c++) xn[(int64_t)t * H + c] = or_round_bf16((double)ht[c] * r * (double)w[c]);
  }
  return OR_OK;
}

/* residual[t][c] = RN_f32(residual[t][c] + out[t][c]) (binary32 add). */
EXPORT void or_residual_add(int64_t n, float* residual, const float* out) {
  for (int64_t i = 0; i < n; i++) residual[i] = residual[i] + out[i];
}

EXPORT int or_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

EXPORT void or_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n);
#else
  (void)n;
#endif
}
