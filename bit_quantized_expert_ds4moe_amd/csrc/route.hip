// route.hip -- router scoring / top-K selection, hash routing and the
// token->expert permutation (gfx950).
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, section
// "MoE FFN 部の中身" (router linear 4096x256 F16, sqrtsoftplus scoring,
// noaux_tc bias used for selection only, top-6, normalised gates, routed
// scaling 1.5; hash routing with a token-id table in layers 0-2).
//
// Routing must be reproducible bit for bit, so each logit is defined as the
// exact dot product rounded once to binary32.  The kernel accumulates it in
// binary64 along a fixed tree of known depth D together with sum|x_c w_c|;
// the classic bound |S - S_hat| <= gamma_D * sum|x_c w_c| (Higham, "Accuracy
// and Stability of Numerical Algorithms", ch. 4) gives an interval that
// contains the exact sum.  sqrtsoftplus is evaluated in binary64 with a
// relative error far below 2^-44, giving an interval for the score, and the
// key interval follows because rounding is monotone.  The selection is
// accepted when every interval is a single binary32 value, or when the chosen
// order holds for every value in the intervals; otherwise the status bit
// DS4MOE_FAULT_UNCERTIFIED is raised.
#include "dev_common.h"

namespace ds4 {

struct RouteArgs {
  const void* x;          // [T][H] bf16 bits or fp32 (ignored with norm)
  int x_dt;
  const float* residual;  // [T][H] fp32: x = RMSNorm(residual) when norm_w set
  const float* norm_w;
  float eps;
  uint16_t* xn_out;       // [T][H] bf16 bits of the normed input (nullable)
  const void* W;          // [E][H] f16 bits or fp32
  int w_dt;
  const float* bias;      // [E]
  int H, E, K, T;
  float scale;
  float4* kbuf;           // [T][E] (key, key_lo, key_hi, score)
  unsigned* counters;     // [T], zero between calls
  int32_t* ids;           // [T][K]
  float* wts;             // [T][K]
  uint32_t* status;
};

__device__ inline double load_x64(const RouteArgs& a, int t, int c, double nscale) {
  if (a.norm_w) {
    double v = (double)a.residual[(size_t)t * a.H + c] * nscale * (double)a.norm_w[c];
    return bf16_bits_to_f64(f64_to_bf16_bits(v));
  }
  if (a.x_dt == DS4MOE_F32) return (double)((const float*)a.x)[(size_t)t * a.H + c];
  return bf16_bits_to_f64(((const uint16_t*)a.x)[(size_t)t * a.H + c]);
}

__device__ inline double load_w64(const RouteArgs& a, int e, int c) {
  if (a.w_dt == DS4MOE_F32) return (double)((const float*)a.W)[(size_t)e * a.H + c];
  return f16_bits_to_f64(((const uint16_t*)a.W)[(size_t)e * a.H + c]);
}

// sqrt(ln(1+e^z)) in binary64, written as sqrt(max(z,0) + ln(1+e^-|z|)).
__device__ inline double sqrtsoftplus64(float zf) {
  double z = (double)zf;
  double az = fabs(z);
  return sqrt(fmax(z, 0.0) + log1p(exp(-az)));
}

// Block-wide fixed-order sum of two doubles over 256 threads (4 waves).
__device__ inline void block_sum2(double& a, double& b, double* sh) {
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
  int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sh[2 * w] = a;
    sh[2 * w + 1] = b;
  }
  __syncthreads();
  a = (sh[0] + sh[2]) + (sh[4] + sh[6]);
  b = (sh[1] + sh[3]) + (sh[5] + sh[7]);
  __syncthreads();
}

__device__ inline bool key_before(float ka, int ea, float kb, int eb) {
  return ka > kb || (ka == kb && ea < eb);
}

// Grid (E, T), 256 threads: block (e, t) scores expert e for token t; the
// last block to finish for token t selects that token's experts.
__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
  __shared__ double sh[8];
  __shared__ int last;
  const int e = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;

  double nscale = 1.0;
  if (a.norm_w) {  // RMSNorm scale, recomputed identically by every block
    double ss = 0.0, dummy = 0.0;
    for (int c = tid; c < a.H; c += 256) {
      double v = (double)a.residual[(size_t)t * a.H + c];
      ss = fma(v, v, ss);
    }
    block_sum2(ss, dummy, sh);
    nscale = 1.0 / sqrt(ss / (double)a.H + (double)a.eps);
    if (e == 0 && a.xn_out)
      for (int c = tid; c < a.H; c += 256)
        a.xn_out[(size_t)t * a.H + c] = (uint16_t)f64_to_bf16_bits(
            (double)a.residual[(size_t)t * a.H + c] * nscale * (double)a.norm_w[c]);
  }

  // Logit: products are exact in binary64; each thread sums its columns in
  // order, then a 6-level wave tree and a 2-level cross-wave tree.
  double acc = 0.0, aabs = 0.0;
  for (int c = tid; c < a.H; c += 256) {
    double p = load_x64(a, t, c, nscale) * load_w64(a, e, c);
    acc += p;
    aabs += fabs(p);
  }
  block_sum2(acc, aabs, sh);

  if (tid == 0) {
    const int depth = (a.H + 255) / 256 + 8;
    const double u = 0x1p-53;
    double bound = (double)(depth + 2) * u * aabs * 1.0009765625;
    // widen by the rounding of acc +- bound itself and an absolute floor
    double b2 = bound + 0x1p-52 * (fabs(acc) + bound) + 0x1p-1070;
    float zm = (float)acc, zl = (float)(acc - b2), zh = (float)(acc + b2);
    double s64 = sqrtsoftplus64(zm);
    float sp = (float)s64;
    const double rel = 0x1p-44;
    double sl64 = (zl == zm) ? s64 : sqrtsoftplus64(zl);
    double sh64 = (zh == zm) ? s64 : sqrtsoftplus64(zh);
    float slo = (float)(sl64 * (1.0 - rel)), shi = (float)(sh64 * (1.0 + rel));
    float b = a.bias[e];
    float key = sp + b, klo = slo + b, khi = shi + b;
    if (key != key) key = klo = khi = -__builtin_huge_valf();  // NaN never wins
    a.kbuf[(size_t)t * a.E + e] = make_float4(key, klo, khi, sp);
  }

  // last-block-done: publish, count, and let the final block select
  __threadfence();
  __syncthreads();
  if (tid == 0) last = (atomicAdd(&a.counters[t], 1u) == (unsigned)(a.E - 1));
  __syncthreads();
  if (!last) return;
  __threadfence();
  if (tid >= 64) return;

  const int lane = tid;
  float kp[4], kl[4], kh[4];
  bool valid[4], sel[4];
  for (int j = 0; j < 4; j++) {
    int ee = lane + 64 * j;
    valid[j] = ee < a.E;
    sel[j] = false;
    float4 v = valid[j] ? a.kbuf[(size_t)t * a.E + ee] : make_float4(0, 0, 0, 0);
    kp[j] = v.x;
    kl[j] = v.y;
    kh[j] = v.z;
  }
  const float NEG = -__builtin_huge_valf();
  int chosen[8];
  int prev = -1;
  bool ok = true;
  // any key with a non-degenerate interval?
  bool wide = false;
  for (int j = 0; j < 4; j++) wide |= valid[j] && (kl[j] != kh[j]);
  wide = __any(wide);
  for (int k = 0; k < a.K; k++) {
    float bk = NEG;
    int be = 1 << 30;
    for (int j = 0; j < 4; j++) {
      int ee = lane + 64 * j;
      if (valid[j] && !sel[j] && key_before(kp[j], ee, bk, be)) {
        bk = kp[j];
        be = ee;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      float ok2 = __shfl_xor(bk, off);
      int oe = __shfl_xor(be, off);
      if (key_before(ok2, oe, bk, be)) {
        bk = ok2;
        be = oe;
      }
    }
    for (int j = 0; j < 4; j++)
      if (lane + 64 * j == be) sel[j] = true;
    if (lane == 0) a.ids[(size_t)t * a.K + k] = be;
    if (k < 8) chosen[k] = be;
    // certification of the order between consecutive selected experts
    if (wide && prev >= 0) {
      float4 pa = a.kbuf[(size_t)t * a.E + prev];
      float4 pb = a.kbuf[(size_t)t * a.E + be];
      if (!(pa.y > pb.z || (pa.y == pb.z && prev < be))) ok = false;
    }
    prev = be;
  }
  if (wide) {
    // the last selected expert must precede every unselected one
    float4 pl = a.kbuf[(size_t)t * a.E + prev];
    for (int j = 0; j < 4; j++) {
      int ee = lane + 64 * j;
      if (valid[j] && !sel[j] && !(pl.y > kh[j] || (pl.y == kh[j] && prev < ee))) ok = false;
    }
    if (__any(!ok) && lane == 0) raise_fault(a.status, DS4MOE_FAULT_UNCERTIFIED);
  }
  if (lane == 0) {
    double ssum = 0.0;
    for (int k = 0; k < a.K; k++) ssum += (double)a.kbuf[(size_t)t * a.E + a.ids[(size_t)t * a.K + k]].w;
    for (int k = 0; k < a.K; k++) {
      double s = (double)a.kbuf[(size_t)t * a.E + a.ids[(size_t)t * a.K + k]].w;
      a.wts[(size_t)t * a.K + k] = (float)((double)a.scale * s / ssum);
    }
    a.counters[t] = 0u;
  }
  (void)chosen;
}

// Hash routing: one thread per token.  Invalid token ids or table rows
// raise a fault bit and route to experts 0..K-1 so that later kernels stay
// in bounds.
__global__ void k_route_hash(const int32_t* tok, const int32_t* table, int vocab, int E, int K, int T,
                             float scale, int32_t* ids, float* wts, uint32_t* status) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int id = tok[t];
  bool good = id >= 0 && id < vocab;
  if (!good) raise_fault(status, DS4MOE_FAULT_BAD_TOKEN);
  bool row_ok = good;
  if (good) {
    const int32_t* row = table + (size_t)id * K;
    for (int k = 0; k < K; k++) {
      int v = row[k];
      if (v < 0 || v >= E) row_ok = false;
      for (int q = 0; q < k; q++)
        if (row[q] == v) row_ok = false;
    }
    if (!row_ok) raise_fault(status, DS4MOE_FAULT_BAD_TABLE);
  }
  float w = (float)((double)scale / (double)K);
  for (int k = 0; k < K; k++) {
    ids[(size_t)t * K + k] = row_ok ? table[(size_t)id * K + k] : k;
    wts[(size_t)t * K + k] = w;
  }
}

// Permutation by a bitonic sort of keys (expert << 15 | pair) in LDS; one
// workgroup of 1024 threads, n = T*K <= 32768.
__global__ __launch_bounds__(1024) void k_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                                  int32_t* offsets, int32_t* perm, int32_t* inv,
                                                  uint32_t* status) {
  extern __shared__ uint32_t keys[];
  __shared__ int cnt[257];
  int tid = threadIdx.x;
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  for (int i = tid; i <= E; i += 1024) cnt[i] = 0;
  bool bad = false;
  for (int i = tid; i < n2; i += 1024) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < n) {
      int e = ids[i];
      if (e < 0 || e >= E) {
        bad = true;
        e = 0;
      }
      key = ((uint32_t)e << 15) | (uint32_t)i;
    }
    keys[i] = key;
  }
  if (bad) raise_fault(status, DS4MOE_FAULT_BAD_ID);
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += 1024) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint32_t a = keys[i], b = keys[ixj];
          bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < n; i += 1024) {
    uint32_t key = keys[i];
    int p = (int)(key & 0x7FFFu);
    perm[i] = p;
    inv[p] = i;
    atomicAdd(&cnt[key >> 15], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; e++) {
      counts[e] = cnt[e];
      offsets[e] = run;
      run += cnt[e];
    }
    offsets[E] = run;
  }
}

}  // namespace ds4
