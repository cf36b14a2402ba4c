// ffn_generic.hip -- shape-generic expert FFN (gfx950): scalar block decode
// and fp32 FMAs, one wave per output row.  Serves fp32 activations, shapes
// other than the V4-Flash expert shape, and any block format; correctness
// path, not a throughput path.
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, section
// "MoE FFN 部の中身".  Formats: DS4C2 = qiita.com/yoshiyakato/items/
// 4678be0e7860ddb444ec, sections 3 and 4; FLOW quantisation table (Q8_0);
// Q4_K: size from the DS4C2 type table, layout of the k-quant family.
#include "dev_common.h"

namespace ds4 {

// Value n of a matrix stored as consecutive blocks of type qt.
__device__ inline float decode_at(int qt, const uint8_t* base, size_t n, const uint8_t* grid) {
  if (qt == DS4MOE_Q8_0) {
    const uint8_t* b = base + (n >> 5) * kQ80Bytes;
    float d = f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8));
    return d * (float)(int8_t)b[2 + (n & 31)];
  }
  const int i = (int)(n & 255);
  if (qt == DS4MOE_Q4_K) {
    const uint8_t* b = base + (n >> 8) * kQ4kBytes;
    const int c = i >> 6, l = i & 31, hi = (i >> 5) & 1, j = i >> 5;
    const int byte = b[16 + 32 * c + l];
    const int q = hi ? byte >> 4 : byte & 15;
    const uint8_t* S = b + 4;
    const int sc = j < 4 ? (S[j] & 63) : ((S[j + 4] & 15) | ((S[j - 4] >> 6) << 4));
    const int m = j < 4 ? (S[j + 4] & 63) : ((S[j + 4] >> 4) | ((S[j] >> 6) << 4));
    const float d = f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8));
    const float dmin = f16_bits_to_f32((uint32_t)b[2] | ((uint32_t)b[3] << 8));
    return d * (float)sc * (float)q - dmin * (float)m;
  }
  if (qt == DS4MOE_Q2_K) {
    const uint8_t* b = base + (n >> 8) * kQ2kBytes;
    int hh = i >> 7, s = (i >> 5) & 3, l = i & 31, j = i >> 4;
    int q = (b[16 + 32 * hh + l] >> (2 * s)) & 3;
    float d = f16_bits_to_f32((uint32_t)b[80] | ((uint32_t)b[81] << 8));
    float dmin = f16_bits_to_f32((uint32_t)b[82] | ((uint32_t)b[83] << 8));
    return d * (float)(b[j] & 15) * (float)q - dmin * (float)(b[j] >> 4);
  }
  const uint8_t* b = base + (n >> 8) * kIq2Bytes;
  int g = i >> 5, k = (i >> 3) & 3, jj = i & 7;
  const uint8_t* gp = b + 2 + 8 * g;
  uint32_t w = (uint32_t)gp[4] | ((uint32_t)gp[5] << 8) | ((uint32_t)gp[6] << 16) | ((uint32_t)gp[7] << 24);
  uint32_t s7 = (w >> (7 * k)) & 0x7F;
  uint32_t s8 = s7 | ((uint32_t)(__popc(s7) & 1) << 7);
  float d = f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8));
  float v = d * (float)(2u * (w >> 28) + 1u) * 0.125f * (float)grid[8 * gp[k] + jj];
  return ((s8 >> jj) & 1u) ? -v : v;
}

__device__ inline float load_act(const void* x, int dt, size_t idx) {
  return dt == DS4MOE_F32 ? ((const float*)x)[idx] : bf16_bits_to_f32(((const uint16_t*)x)[idx]);
}

struct GenericArgs {
  const void* x;
  int x_dt;
  int H, I, E, K, T;
  // routed experts
  int qt_g, qt_u, qt_d;
  const uint8_t *gate, *up, *down, *grid;
  // shared expert (nullable)
  int sh_I, sh_qt_g, sh_qt_u, sh_qt_d;
  const uint8_t *sh_gate, *sh_up, *sh_down, *sh_grid;
  const int32_t* ids;
  const float* wts;
  float* h;   // [T*K + T][max(I, sh_I)]
  float* y;   // [T*K + T][H]
  float* out;
  float* residual;
  int n_sh;   // T if shared present else 0
  uint32_t* status;
};

// pair p < T*K: routed (token p/K, expert ids[p]); p >= T*K: shared expert of token p-T*K
__device__ inline bool pair_info(const GenericArgs& a, int p, int& tok, int& e) {
  if (p < a.T * a.K) {
    tok = p / a.K;
    e = a.ids[p];
    if (e < 0 || e >= a.E) {
      raise_fault(a.status, DS4MOE_FAULT_BAD_ID);
      e = 0;
    }
    return false;
  }
  tok = p - a.T * a.K;
  e = 0;
  return true;
}

// Grid (ceil(Imax/4), n_pairs), 256 threads: one wave per (pair, row).
__global__ __launch_bounds__(256) void k_generic_gateup(GenericArgs a) {
  const int p = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  int tok, e;
  bool sh = pair_info(a, p, tok, e);
  const int I = sh ? a.sh_I : a.I;
  if (i >= I) return;
  const int qg = sh ? a.sh_qt_g : a.qt_g, qu = sh ? a.sh_qt_u : a.qt_u;
  const uint8_t* G = sh ? a.sh_gate : a.gate;
  const uint8_t* U = sh ? a.sh_up : a.up;
  const uint8_t* grid = sh ? a.sh_grid : a.grid;
  const size_t row0 = ((size_t)e * I + i) * (size_t)a.H;
  float g = 0.0f, u = 0.0f;
  for (int c = lane; c < a.H; c += 64) {
    float xv = load_act(a.x, a.x_dt, (size_t)tok * a.H + c);
    g = fmaf(decode_at(qg, G, row0 + c, grid), xv, g);
    u = fmaf(decode_at(qu, U, row0 + c, grid), xv, u);
  }
  g = wave_sum(g);
  u = wave_sum(u);
  if (lane == 0) a.h[(size_t)p * max(a.I, a.sh_I) + i] = silu(g) * u;
}

// Grid (H/4, n_pairs): y[p][r] = W_down[e][r] . h[p]
__global__ __launch_bounds__(256) void k_generic_down(GenericArgs a) {
  const int p = blockIdx.y, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.H) return;
  int tok, e;
  bool sh = pair_info(a, p, tok, e);
  const int I = sh ? a.sh_I : a.I;
  const int qd = sh ? a.sh_qt_d : a.qt_d;
  const uint8_t* D = sh ? a.sh_down : a.down;
  const uint8_t* grid = sh ? a.sh_grid : a.grid;
  const size_t row0 = ((size_t)e * a.H + r) * (size_t)I;
  const float* hp = a.h + (size_t)p * max(a.I, a.sh_I);
  float acc = 0.0f;
  for (int c = lane; c < I; c += 64) acc = fmaf(decode_at(qd, D, row0 + c, grid), hp[c], acc);
  acc = wave_sum(acc);
  if (lane == 0) a.y[(size_t)p * a.H + r] = acc;
}

// out[t][r] = sum_k w[t][k] y[t*K+k][r] (+ y_shared[t][r]) (+ residual)
__global__ void k_generic_combine(GenericArgs a) {
  const size_t n = (size_t)a.T * a.H;
  size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  int t = (int)(idx / a.H), r = (int)(idx % a.H);
  float acc = 0.0f;
  for (int k = 0; k < a.K; k++) acc = fmaf(a.wts[t * a.K + k], a.y[((size_t)t * a.K + k) * a.H + r], acc);
  if (a.n_sh) acc += a.y[((size_t)a.T * a.K + t) * a.H + r];
  if (a.residual) a.residual[idx] += acc;
  else a.out[idx] = acc;
}

}  // namespace ds4
