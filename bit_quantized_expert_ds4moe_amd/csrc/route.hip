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
// DS4MOE_FAULT_UNCERTIFIED is raised.  Scoring and selection are two kernels:
// the kernel boundary publishes the scores without any in-kernel fence.
#include "dev_common.h"
#include "ssp64.h"

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

// Order-preserving map of a binary32 key to uint32, combined with the expert
// index so that a larger composite means "earlier in the selection order":
// higher key first, then lower index.
__device__ inline uint64_t sel_composite(float key, int e) {
  uint32_t u = __float_as_uint(key);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFF - e);
}

template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ inline uint64_t readlane_u64(uint64_t v, int lane) {
  uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));
  v = umax64(v, dpp_u64<0x4E>(v));
  v = umax64(v, dpp_u64<0x141>(v));
  v = umax64(v, dpp_u64<0x140>(v));
  return umax64(umax64(readlane_u64(v, 0), readlane_u64(v, 16)),
                umax64(readlane_u64(v, 32), readlane_u64(v, 48)));
}
__device__ inline float readlane_f32(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

constexpr int kMaxRouteK = 16;

// Scoring.  Grid (E, T), 256 threads: block (e, t) computes the logit, score
// and key interval of expert e for token t.  VEC (hidden % 2048 == 0, fp16
// router, bf16 or normalised input): thread t owns columns 8t..8t+7 of every
// 2048-column slab and reads them with 16-byte loads; otherwise thread t owns
// columns t, t+256, ...  Either way each thread sums its products in column
// order before the fixed reduction tree (depth hidden/256 + 8).  The kernel is
// specialised so that the batch-1 variant carries no unused code: its blocks
// run through their code once, and instruction fetch is on the critical path.
template <bool NORM, bool VEC>
__global__ __launch_bounds__(256) void k_route_score(RouteArgs a) {
  __shared__ double sh[8];
  const int e = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  constexpr int kMaxSlab = 2;  // VEC: hidden <= 4096

  uint4 wv[kMaxSlab];
  if (VEC) {  // router-weight loads first: their latency overlaps the input
    const uint4* wp = (const uint4*)((const uint16_t*)a.W + (size_t)e * a.H);
#pragma unroll
    for (int j = 0; j < kMaxSlab; j++)
      if (j < a.H / 2048) wv[j] = wp[256 * j + tid];
  }
  // Normalised input: the residual and norm weight of the thread's own
  // columns are loaded once, up front; the columns of all threads cover the
  // row exactly once, so the sum of squares comes from the same registers.
  float rr[kMaxSlab][8], nw[kMaxSlab][8];
  double nscale = 1.0;
  if (NORM && VEC) {
#pragma unroll
    for (int j = 0; j < kMaxSlab; j++) {
      if (j >= a.H / 2048) break;
      const float4* rp = (const float4*)(a.residual + (size_t)t * a.H) + 512 * j + 2 * tid;
      const float4* np = (const float4*)a.norm_w + 512 * j + 2 * tid;
      const float4 r0 = rp[0], r1 = rp[1], n0 = np[0], n1 = np[1];
      rr[j][0] = r0.x; rr[j][1] = r0.y; rr[j][2] = r0.z; rr[j][3] = r0.w;
      rr[j][4] = r1.x; rr[j][5] = r1.y; rr[j][6] = r1.z; rr[j][7] = r1.w;
      nw[j][0] = n0.x; nw[j][1] = n0.y; nw[j][2] = n0.z; nw[j][3] = n0.w;
      nw[j][4] = n1.x; nw[j][5] = n1.y; nw[j][6] = n1.z; nw[j][7] = n1.w;
    }
    double ss = 0.0, dummy = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxSlab; j++) {
      if (j >= a.H / 2048) break;
#pragma unroll
      for (int u = 0; u < 8; u++) ss = fma((double)rr[j][u], (double)rr[j][u], ss);
    }
    block_sum2(ss, dummy, sh);
    nscale = 1.0 / sqrt(ss / (double)a.H + (double)a.eps);
  } else if (NORM) {  // generic shapes: strided columns
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

  double acc = 0.0, aabs = 0.0;
  if (VEC) {
#pragma unroll
    for (int j = 0; j < kMaxSlab; j++) {
      if (j >= a.H / 2048) break;
      uint32_t xx[4];
      if (!NORM) {
        const uint4 xv = ((const uint4*)((const uint16_t*)a.x + (size_t)t * a.H))[256 * j + tid];
        xx[0] = xv.x; xx[1] = xv.y; xx[2] = xv.z; xx[3] = xv.w;
      } else {
        // rare results outside the normal bfloat16 range take the general
        // rounding in a separate pass (no call in the common path)
        uint32_t bb[8];
        bool all_ok = true;
#pragma unroll
        for (int u = 0; u < 8; u++) {
          bool ok;
          bb[u] = f64_to_bf16_bits_fast((double)rr[j][u] * nscale * (double)nw[j][u], ok);
          all_ok &= ok;
        }
        if (!all_ok)
          for (int u = 0; u < 8; u++) {
            bool ok;
            (void)f64_to_bf16_bits_fast((double)rr[j][u] * nscale * (double)nw[j][u], ok);
            if (!ok) bb[u] = f64_to_bf16_bits_general((double)rr[j][u] * nscale * (double)nw[j][u]);
          }
#pragma unroll
        for (int m = 0; m < 4; m++) xx[m] = bb[2 * m] | (bb[2 * m + 1] << 16);
        if (e == 0 && a.xn_out)
          ((uint4*)(a.xn_out + (size_t)t * a.H))[256 * j + tid] = make_uint4(xx[0], xx[1], xx[2], xx[3]);
      }
      const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const uint32_t sh16 = 16 * (u & 1);
        const double xd = bf16_bits_to_f64((xx[u >> 1] >> sh16) & 0xFFFFu);
        const double p = xd * f16_bits_to_f64((ww[u >> 1] >> sh16) & 0xFFFFu);
        acc += p;
        aabs += fabs(p);
      }
    }
  } else {
    for (int c = tid; c < a.H; c += 256) {
      double p = load_x64(a, t, c, nscale) * load_w64(a, e, c);
      acc += p;
      aabs += fabs(p);
    }
  }
  block_sum2(acc, aabs, sh);

  if (tid == 0) {
    const int depth = (a.H + 255) / 256 + 8;
    double bound = (double)(depth + 2) * 0x1p-53 * aabs * 1.0009765625;
    // widen by the rounding of acc +- bound itself and an absolute floor
    double b2 = bound + 0x1p-52 * (fabs(acc) + bound) + 0x1p-1070;
    float zm = (float)acc, zl = (float)(acc - b2), zh = (float)(acc + b2);
    double s64 = ssp64(zm);
    double sl64 = s64, sh64 = s64;
    if (zl != zm || zh != zm) {  // rare: the logit itself is not certified
      sl64 = ssp64(zl);
      sh64 = ssp64(zh);
    }
    const double rel = 0x1p-40;  // far above the error of ssp64
    float sp = (float)s64;
    float slo = (float)(sl64 * (1.0 - rel)), shi = (float)(sh64 * (1.0 + rel));
    float b = a.bias[e];
    float key = sp + b, klo = slo + b, khi = shi + b;
    if (key != key) key = klo = khi = -__builtin_huge_valf();  // NaN never wins
    a.kbuf[(size_t)t * a.E + e] = make_float4(key, klo, khi, sp);
  }
}

// Order-preserving map of a binary32 key to uint32 (larger key, larger code;
// keys are never NaN or -0 here), 0 marking an expert out of the running.
__device__ inline uint32_t key_order(float key) {
  const uint32_t u = __float_as_uint(key);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Maximum over the 64 lanes, left in every lane: DPP maxima inside rows of
// 16, then the two lane-swap steps across rows (no scalar round trip).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max((uint32_t)h[0], (uint32_t)h[1]);
  auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}

// Top-K selection for one token by one wave, from the E <= 256 key intervals
// of k_route_score: K rounds of "largest key, lowest expert index among
// equal keys" (a wave maximum of the key codes, then the first expert whose
// code equals it).  Lane k < K records the k-th expert; the winners' scores
// and intervals are read back afterwards (one load per lane, from lines the
// wave has just read), so a round carries no per-winner lookups.  On return
// lane k < K holds slot k: expert id in e_out and gate in w_out.  When report
// is set, an uncertified order raises the fault bit.  Deterministic: every
// wave that runs it on the same keys gets the same answer.
__device__ inline void select_wave(const float4* kb, int E, int K, float scale, uint32_t* status,
                                   bool report, int& e_out, float& w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t ko[4];
  float kh[4];
  bool wide = false;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int ee = lane + 64 * j;
    const float4 v = ee < E ? kb[ee] : make_float4(0, 0, 0, 0);
    ko[j] = ee < E ? key_order(v.x) : 0u;
    kh[j] = v.z;
    wide |= ee < E && (v.y != v.z);
  }
  int e_sel = 0;  // lane k: the k-th winner
  for (int k = 0; k < K; k++) {
    const uint32_t m = wave_max_u32(max(max(ko[0], ko[1]), max(ko[2], ko[3])));
    int be = 0;
#pragma unroll
    for (int j = 3; j >= 0; j--) {
      const unsigned long long bal = __ballot(ko[j] == m);
      if (bal) be = 64 * j + __ffsll((long long)bal) - 1;
    }
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (lane + 64 * j == be) ko[j] = 0u;
    if (lane == k) e_sel = be;
  }
  const float4 win = lane < K ? kb[e_sel] : make_float4(0, 0, 0, 0);  // key, lo, hi, score
  if (__any(wide)) {
    bool ok = true;
    // consecutive winners: the interval of winner k-1 lies above that of k
    const float plo = __shfl_up(win.y, 1);
    const int pe = __shfl_up(e_sel, 1);
    if (lane >= 1 && lane < K && !(plo > win.z || (plo == win.z && pe < e_sel))) ok = false;
    // the last winner precedes every unselected expert
    const float last_lo = readlane_f32(win.y, K - 1);
    const int last_e = __builtin_amdgcn_readlane(e_sel, K - 1);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int ee = lane + 64 * j;
      if (ee < E && ko[j] != 0u && !(last_lo > kh[j] || (last_lo == kh[j] && last_e < ee)))
        ok = false;
    }
    if (__any(!ok) && lane == 0 && report) raise_fault(status, DS4MOE_FAULT_UNCERTIFIED);
  }
  double ssum = 0.0;
  for (int k = 0; k < K; k++) ssum += (double)readlane_f32(win.w, k);
  e_out = lane < K ? e_sel : 0;
  w_out = lane < K ? (float)((double)scale * (double)win.w / ssum) : 0.0f;
}

// Selection kernel.  Grid T, one wave per token: reads the key intervals
// written by k_route_score (visible at the kernel boundary), picks the top K
// and writes ids and gates.
__global__ __launch_bounds__(64) void k_route_select(RouteArgs a) {
  const int t = blockIdx.x, lane = threadIdx.x;
  int e;
  float w;
  select_wave(a.kbuf + (size_t)t * a.E, a.E, a.K, a.scale, a.status, true, e, w);
  if (lane < a.K) {
    a.ids[(size_t)t * a.K + lane] = e;
    a.wts[(size_t)t * a.K + lane] = w;
  }
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

// Permutation by a stable counting sort in one workgroup of 1024 threads
// (n = T*K <= 32768, E <= 256).  The expert ids are staged in LDS as bytes;
// 64 chunk owners count their contiguous run of pairs per expert; an
// exclusive scan over chunks (per expert) and over experts gives every
// (chunk, expert) its first position; each owner then places its pairs in
// order.  The result is the canonical order: by expert, then by pair index.
// Invalid ids raise a fault bit and are treated as expert 0.
constexpr int kPermChunks = 64;
constexpr int kPermMax = 32768;

__global__ __launch_bounds__(1024) void k_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                                  int32_t* offsets, int32_t* perm, int32_t* inv,
                                                  uint32_t* status) {
  __shared__ int tab[kPermChunks * 256];  // [chunk][expert]: counts, then first positions
  __shared__ uint8_t eid[kPermMax];
  __shared__ int base[257];
  const int tid = threadIdx.x;
  for (int i = tid; i < kPermChunks * 256; i += 1024) tab[i] = 0;
  bool bad = false;
  for (int i = tid; i < n; i += 1024) {
    int e = ids[i];
    if (e < 0 || e >= E) {
      bad = true;
      e = 0;
    }
    eid[i] = (uint8_t)e;
  }
  if (bad) raise_fault(status, DS4MOE_FAULT_BAD_ID);
  __syncthreads();
  const int per = (n + kPermChunks - 1) / kPermChunks;
  if (tid < kPermChunks) {
    const int i0 = tid * per, i1 = min(n, i0 + per);
    for (int i = i0; i < i1; i++) tab[tid * 256 + eid[i]]++;
  }
  __syncthreads();
  if (tid < E) {  // per expert: exclusive prefix over chunks, total
    int run = 0;
    for (int c = 0; c < kPermChunks; c++) {
      const int v = tab[c * 256 + tid];
      tab[c * 256 + tid] = run;
      run += v;
    }
    base[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {  // exclusive scan over experts
    int run = 0;
    for (int e = 0; e < E; e++) {
      const int c = base[e];
      counts[e] = c;
      offsets[e] = run;
      base[e] = run;
      run += c;
    }
    offsets[E] = run;
  }
  __syncthreads();
  if (tid < kPermChunks) {
    const int i0 = tid * per, i1 = min(n, i0 + per);
    for (int i = i0; i < i1; i++) {
      const int e = eid[i];
      const int pos = base[e] + tab[tid * 256 + e]++;
      perm[pos] = i;
      inv[i] = pos;
    }
  }
}

}  // namespace ds4
