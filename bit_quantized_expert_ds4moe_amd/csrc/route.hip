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
// order holds for every value in the intervals.  Otherwise (rare: a logit or
// score within the error bound of a binary32 rounding point, next to the
// selection's cut) the selecting wave recomputes the keys of every expert
// that could still be selected exactly: the logit as an integer-limb sum of
// the exact products (integer additions are associative, so any summation
// order gives the same bits), rounded once; the score in double-double
// arithmetic with its rounding decided against an error bound of 2^-90.
// Scoring and selection are two kernels: the kernel boundary publishes the
// scores without any in-kernel fence.
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
  // Few-token layer calls (T*K <= kSelItemsMax; nullable: not built): the
  // selection runs as one workgroup, wave t selecting token t, which then
  // also sorts the pairs p = tK + k by (expert, p) and lists one work item
  // per expert, as the grouped path's permutation and item list do.
  int32_t* perm;          // [T*K] sorted position -> pair
  int32_t* items;         // [n][3]: expert, first sorted position, pairs
  int32_t* n_items;       // [2]: items, items of at most 16 pairs
};
constexpr int kSelItemsMax = 128;

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

// Where the router input and weights of one token live, for the exact
// recomputation of a logit by the selecting wave.
struct RouteSrc {
  const void* x;      // the token's router input row: bf16 bits or fp32
  int x_dt;
  const void* W;      // [E][H] f16 bits or fp32
  int w_dt;
  const float* bias;  // [E]
  int H;
};

// ---- exact logit --------------------------------------------------------
// Every product of a router input and a router weight is a product of two
// binary32 values (bf16 and f16 values are binary32 values): an integer
// m < 2^48 times 2^e, e >= -298.  A wave adds the products into a fixed-point
// accumulator of kXLimbs limbs of 32 bits (limb j weighs 2^(32j - 298)), held
// in int64 so that carries wait until the end (4096 products of < 2^32 per
// limb stay below 2^44), sums the lanes' limbs, propagates the carries and
// rounds the total once to binary32 (nearest, ties to even).
constexpr int kXLimbs = 18;   // bits 0 .. 575: products reach bit 554, sums 12 more
constexpr int kXBase = 298;

// binary32 bit pattern -> m * 2^e with m < 2^24; false for NaN / infinity
__device__ inline bool f32_parts(uint32_t u, uint32_t& m, int& e) {
  const uint32_t ex = (u >> 23) & 0xFFu, fr = u & 0x7FFFFFu;
  m = ex ? (fr | 0x800000u) : fr;
  e = ex ? (int)ex - 150 : -149;
  return ex != 0xFFu;
}

// limb j of a (static) limb array, for a run-time j (out of range: 0)
__device__ inline int64_t limb_at(const int64_t (&L)[kXLimbs], int j) {
  int64_t v = 0;
#pragma unroll
  for (int i = 0; i < kXLimbs; i++) v = (i == j) ? L[i] : v;
  return v;
}

__device__ inline void limbs_carry(int64_t (&L)[kXLimbs]) {
#pragma unroll
  for (int i = 0; i < kXLimbs - 1; i++) {
    const int64_t c = L[i] >> 32;  // arithmetic: floor division by 2^32
    L[i] -= c * 4294967296LL;
    L[i + 1] += c;
  }
}

// RN_f32 of sum_c x[c] * W[e][c], computed by one wave (the result in every
// lane).  ok is false if an input is NaN or infinite.
__device__ __noinline__ float exact_logit_wave(RouteSrc src, int e, bool& ok) {
  const int lane = threadIdx.x & 63;
  int64_t L[kXLimbs];
#pragma unroll
  for (int i = 0; i < kXLimbs; i++) L[i] = 0;
  bool finite = true;
  for (int c = lane; c < src.H; c += 64) {
    const uint32_t xu = src.x_dt == DS4MOE_F32
                            ? ((const uint32_t*)src.x)[c]
                            : (uint32_t)((const uint16_t*)src.x)[c] << 16;
    const size_t wi = (size_t)e * src.H + c;
    const uint32_t wu = src.w_dt == DS4MOE_F32
                            ? ((const uint32_t*)src.W)[wi]
                            : __float_as_uint(f16_bits_to_f32(((const uint16_t*)src.W)[wi]));
    uint32_t mx, mw;
    int ex, ew;
    const bool fx = f32_parts(xu, mx, ex), fw = f32_parts(wu, mw, ew);
    finite = finite && fx && fw;
    const uint64_t P = (uint64_t)mx * mw;
    if (P == 0) continue;
    const int o = ex + ew + kXBase;  // >= 0
    const int j = o >> 5, sft = o & 31;
    const uint64_t t0 = (uint64_t)(uint32_t)P << sft;
    const uint64_t t1 = ((P >> 32) << sft) + (t0 >> 32);
    const int64_t p0 = (int64_t)(uint32_t)t0, p1 = (int64_t)(uint32_t)t1, p2 = (int64_t)(t1 >> 32);
    const bool neg = ((xu ^ wu) >> 31) != 0;
#pragma unroll
    for (int i = 0; i < kXLimbs; i++) {
      const int64_t add = i == j ? p0 : i == j + 1 ? p1 : i == j + 2 ? p2 : 0;
      L[i] += neg ? -add : add;
    }
  }
  ok = !__any(!finite);
  // the lanes' sums (exact integer additions, any order)
#pragma unroll
  for (int i = 0; i < kXLimbs; i++) {
    int64_t v = L[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    L[i] = v;
  }
  limbs_carry(L);
  const bool negative = L[kXLimbs - 1] < 0;
  if (negative) {
#pragma unroll
    for (int i = 0; i < kXLimbs; i++) L[i] = -L[i];
    limbs_carry(L);
  }
  // the magnitude N = sum L[i] 2^(32 i), every limb now in [0, 2^32)
  int top = -1;
#pragma unroll
  for (int i = 0; i < kXLimbs; i++)
    if (L[i] != 0) top = 32 * i + 31 - __builtin_clz((uint32_t)L[i]);
  if (top < 0) return 0.0f;
  int q = max(top - 23, 149);  // the unit of the last kept bit (2^-149: subnormals)
  auto bits_at = [&](int b) -> uint64_t {  // N >> b, low 64 bits
    const int j = b >> 5, sft = b & 31;
    const uint64_t w0 = (uint64_t)limb_at(L, j), w1 = (uint64_t)limb_at(L, j + 1),
                   w2 = (uint64_t)limb_at(L, j + 2);
    const uint64_t lo = w0 | (w1 << 32);
    return sft ? ((lo >> sft) | (w2 << (64 - sft))) : lo;
  };
  uint32_t M = (uint32_t)bits_at(q);  // < 2^24
  const uint32_t rbit = (uint32_t)bits_at(q - 1) & 1u;
  bool sticky = false;
  const int sb = q - 1;  // bits below sb
#pragma unroll
  for (int i = 0; i < kXLimbs; i++) {
    const int lo = 32 * i;
    const uint32_t mask = sb >= lo + 32 ? 0xFFFFFFFFu : sb <= lo ? 0u : ((1u << (sb - lo)) - 1u);
    sticky |= ((uint32_t)L[i] & mask) != 0u;
  }
  if (rbit && (sticky || (M & 1u))) M++;
  if (M == (1u << 24)) {
    M >>= 1;
    q++;
  }
  float r = q - kXBase > 104 ? __builtin_huge_valf() : ldexpf((float)M, q - kXBase);
  return negative ? -r : r;
}


// RMSNorm scale of token t for hidden % 2048 == 0, up to 4096, with 256
// threads: thread tid loads the residual and norm weight of columns
// 2048 j + 8 tid .. +7 (into rr, nw; rms_load_vec) and the block sums the
// squares along a fixed tree in binary64 (rms_scale_of); returns
// 1 / sqrt(mean + eps).  Every block that calls them for a token gets the
// same bits.  Callers request other data between the two.
__device__ inline void rms_load_vec(const RouteArgs& a, int t, float (&rr)[2][8], float (&nw)[2][8]) {
  const int tid = threadIdx.x;
  const int nslab = a.H / 2048;  // 1 or 2; the loads are unconditional (see route_score_block)
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int js = min(j, nslab - 1);
    const float4* rp = (const float4*)(a.residual + (size_t)t * a.H) + 512 * js + 2 * tid;
    const float4* np = (const float4*)a.norm_w + 512 * js + 2 * tid;
    const float4 r0 = rp[0], r1 = rp[1], n0 = np[0], n1 = np[1];
    rr[j][0] = r0.x; rr[j][1] = r0.y; rr[j][2] = r0.z; rr[j][3] = r0.w;
    rr[j][4] = r1.x; rr[j][5] = r1.y; rr[j][6] = r1.z; rr[j][7] = r1.w;
    nw[j][0] = n0.x; nw[j][1] = n0.y; nw[j][2] = n0.z; nw[j][3] = n0.w;
    nw[j][4] = n1.x; nw[j][5] = n1.y; nw[j][6] = n1.z; nw[j][7] = n1.w;
  }
}
__device__ inline double rms_scale_of(const RouteArgs& a, double* sh, const float (&rr)[2][8]) {
  double ss = 0.0, dummy = 0.0;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    if (j >= a.H / 2048) break;
#pragma unroll
    for (int u = 0; u < 8; u++) ss = fma((double)rr[j][u], (double)rr[j][u], ss);
  }
  block_sum2(ss, dummy, sh);
  return 1.0 / sqrt(ss / (double)a.H + (double)a.eps);
}

// Scoring.  Grid (E, T), 256 threads: block (e, t) computes the logit, score
// and key interval of expert e for token t.  VEC (hidden % 2048 == 0, fp16
// router, bf16 or normalised input): thread t owns columns 8t..8t+7 of every
// 2048-column slab and reads them with 16-byte loads; otherwise thread t owns
// columns t, t+256, ...  Either way each thread sums its products in column
// order before the fixed reduction tree (depth hidden/256 + 8).  The kernel is
// specialised so that the batch-1 variant carries no unused code: its blocks
// run through their code once, and instruction fetch is on the critical path.
template <bool NORM, bool VEC>
__device__ inline void route_score_block(const RouteArgs& a, int e, int t) {
  __shared__ double sh[8];
  const int tid = threadIdx.x;
  constexpr int kMaxSlab = 2;  // VEC: hidden <= 4096

  // VEC: every load up front and unconditional (with one slab, the second
  // load repeats the first and is not used), so that all of them are in
  // flight together: loads issued inside the slab loop went out one round
  // trip after another
  const int nslab = VEC ? a.H / 2048 : 0;  // 1 or 2
  // the expert's bias, requested now through the scalar cache (read at the
  // end, it was a round trip of its own)
  const float bias_e = __int_as_float(load_scalar_i32((const int32_t*)a.bias, e));
  // Normalised input: the residual and norm weight of the thread's own
  // columns, requested before the router weights so that the norm's wait
  // (the vector memory counter retires in order) does not wait for them; the
  // columns of all threads cover the row exactly once, so the sum of squares
  // comes from the same registers.
  float rr[kMaxSlab][8], nw[kMaxSlab][8];
  if (NORM && VEC) rms_load_vec(a, t, rr, nw);
  uint4 wv[kMaxSlab], xv[kMaxSlab];
  if (VEC) {  // router weights, then (not normalised) the input
    const uint4* wp = (const uint4*)((const uint16_t*)a.W + (size_t)e * a.H);
#pragma unroll
    for (int j = 0; j < kMaxSlab; j++) wv[j] = wp[256 * min(j, nslab - 1) + tid];
    if (!NORM) {
      const uint4* xp = (const uint4*)((const uint16_t*)a.x + (size_t)t * a.H);
#pragma unroll
      for (int j = 0; j < kMaxSlab; j++) xv[j] = xp[256 * min(j, nslab - 1) + tid];
      // an empty asm that reads one word of every load, so that the
      // compiler neither sinks the second slab's loads into the branch that
      // uses them nor issues them after the first slab's wait
      asm volatile("" ::"v"(wv[0].x), "v"(wv[1].x), "v"(xv[0].x), "v"(xv[1].x), "s"(bias_e));
    }
  }
  double nscale = 1.0;
  if (NORM && VEC) {
    nscale = rms_scale_of(a, sh, rr);
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
        xx[0] = xv[j].x; xx[1] = xv[j].y; xx[2] = xv[j].z; xx[3] = xv[j].w;
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
    const float b = bias_e;
    float key = sp + b, klo = slo + b, khi = shi + b;
    if (key != key) key = klo = khi = -__builtin_huge_valf();  // NaN never wins
    a.kbuf[(size_t)t * a.E + e] = make_float4(key, klo, khi, sp);
  }
}

template <bool NORM, bool VEC>
__global__ __launch_bounds__(256) void k_route_score(RouteArgs a) {
  route_score_block<NORM, VEC>(a, blockIdx.x, blockIdx.y);
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

// K rounds of "largest key, lowest expert index among equal keys" over the
// key codes ko (expert lane + 64 j in slot j; 0 = out of the running): a
// wave maximum of the codes, then the first expert whose code equals it.
// Lane k < K returns the k-th winner; the winners' codes are cleared.
__device__ inline int select_rounds(uint32_t (&ko)[4], int K) {
  const int lane = threadIdx.x & 63;
  int e_sel = 0;
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
  return e_sel;
}

// Descending sorting network on four values (five compare-exchanges).
__device__ inline void sort4_desc(uint32_t (&c)[4]) {
  auto cx = [](uint32_t& a, uint32_t& b) {
    const uint32_t hi = max(a, b), lo = min(a, b);
    a = hi;
    b = lo;
  };
  cx(c[0], c[1]);
  cx(c[2], c[3]);
  cx(c[0], c[2]);
  cx(c[1], c[3]);
  cx(c[1], c[2]);
}

// The same K rounds on packed codes: the upper 24 bits of the key code and
// 255 - expert in the low byte, so that every code is unique and carries its
// expert.  Each lane keeps its four codes sorted, so a round is one wave
// maximum over the lanes' heads and a pop in the winning lane (no ballots,
// no scalar search).  The packed order is the exact one unless two codes that
// decide the result share their upper 24 bits: two winners, or the last
// winner and an expert left out.  Then the function returns false and the
// caller reruns select_rounds on the full codes.  Otherwise lane k < K
// returns the k-th winner in e_sel.
__device__ inline bool select_rounds_packed(const uint32_t (&ko)[4], int K, int& e_sel) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4];
#pragma unroll
  for (int j = 0; j < 4; j++)
    c[j] = ko[j] ? ((ko[j] & 0xFFFFFF00u) | (uint32_t)(255 - (lane + 64 * j))) : 0u;
  sort4_desc(c);
  uint32_t mine = 0u, m = 0u, prev = 0u;
  bool clash = false;
  for (int k = 0; k < K; k++) {
    m = wave_max_u32(c[0]);
    clash |= k > 0 && (m >> 8) == (prev >> 8);
    prev = m;
    const bool pop = c[0] == m;
    c[0] = pop ? c[1] : c[0];
    c[1] = pop ? c[2] : c[1];
    c[2] = pop ? c[3] : c[2];
    c[3] = pop ? 0u : c[3];
    if (lane == k) mine = m;
  }
  // a head left behind with the last winner's upper bits (packed codes are
  // never 0 for a real expert, so 0 never matches)
  clash |= c[0] != 0u && (c[0] >> 8) == (m >> 8);
  e_sel = 255 - (int)(mine & 0xFFu);
  return !__any(clash);
}

// Exact selection among the experts that the key intervals cannot rule out
// (upper end at or above `floor`, the lowest lower end among the approximate
// winners: every other expert lies below K of them for sure).  Each
// candidate's key is recomputed exactly (exact logit, double-double score);
// K rounds over the exact keys give the winners.  Lane k < K returns the
// k-th winner in e_sel and its score in s_sel.  A score too close to a
// rounding point for double-double (never seen; the oracle stops there too)
// raises DS4MOE_FAULT_UNCERTIFIED when report is set.
__device__ __noinline__ void select_exact(const float4* kb, int E, int K, float floor,
                                          RouteSrc src, uint32_t* status, bool report, int& e_out,
                                          float& s_out) {
  const int lane = threadIdx.x & 63;
  uint32_t ko[4];
  float sc[4];
  unsigned long long cand[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int ee = lane + 64 * j;
    cand[j] = __ballot(ee < E && kb[ee < E ? ee : 0].z >= floor);
    ko[j] = 0u;
    sc[j] = 0.0f;
  }
  bool fault = false;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    unsigned long long m = cand[j];
    while (m) {
      const int l = __ffsll((long long)m) - 1;
      m &= m - 1;
      const int e = 64 * j + l;
      bool fin;
      const float z = exact_logit_wave(src, e, fin);
      bool dec = true;
      float s = fin ? dd_round_f32(ssp_dd(z), 0x1p-90, dec) : __builtin_nanf("");
      fault |= !dec;
      float key = s + src.bias[e];
      if (key != key) key = -__builtin_huge_valf();  // NaN never wins
      if (lane == l) {
        ko[j] = key_order(key);
        sc[j] = s;
      }
    }
  }
  if (fault && lane == 0 && report) raise_fault(status, DS4MOE_FAULT_UNCERTIFIED);
  const int e_sel = select_rounds(ko, K);
  // the winner's score from the lane that holds it
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float v = __shfl(sc[j], e_sel & 63);
    s = (e_sel >> 6) == j ? v : s;
  }
  e_out = e_sel;
  s_out = s;
}

// Top-K selection for one token by one wave, from the E <= 256 key intervals
// of k_route_score, in two parts so that a caller can request expert weights
// between them.  select_ids: the rounds on the approximate keys
// (select_rounds_packed, or select_rounds on the full codes when packed codes
// clash); when an interval is wider than one binary32 value, the winners'
// intervals are read back and the order is certified, else the selection is
// redone on exact keys (select_exact).  Lane k < K holds the k-th expert.
// select_gate: lane k < K gets the gate of its expert, from the score the
// exact pass computed or else the one k_route_score stored (read back from
// lines the wave has just read).  Deterministic: every wave that runs them on
// the same inputs gets the same answer.
struct SelIds {
  int e;       // lane k < K: the k-th expert
  float s;     // its score when `exact`
  bool exact;  // wave-uniform: the exact pass ran
};

__device__ inline SelIds select_ids(const float4* kb, int E, int K, uint32_t* status, bool report,
                                    const RouteSrc& src) {
  const int lane = threadIdx.x & 63;
  uint32_t ko[4];
  float kh[4];
  bool wide = false;
  // four unconditional loads (indices past E read entry E - 1 and are then
  // masked), so that they go out together: loads in branches of their own
  // were each preceded by a wait for the one before
  float4 v[4];
#pragma unroll
  for (int j = 0; j < 4; j++) v[j] = kb[min(lane + 64 * j, E - 1)];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int ee = lane + 64 * j;
    ko[j] = ee < E ? key_order(v[j].x) : 0u;
    kh[j] = v[j].z;
    wide |= ee < E && (v[j].y != v[j].z);
  }
  SelIds r{0, 0.0f, false};
  if (!select_rounds_packed(ko, K, r.e)) r.e = select_rounds(ko, K);
  if (__any(wide)) {
    const float4 win = lane < K ? kb[r.e] : make_float4(0, 0, 0, 0);  // key, lo, hi, score
    bool ok = true;
    // consecutive winners: the interval of winner k-1 lies above that of k
    const float plo = __shfl_up(win.y, 1);
    const int pe = __shfl_up(r.e, 1);
    if (lane >= 1 && lane < K && !(plo > win.z || (plo == win.z && pe < r.e))) ok = false;
    // the last winner precedes every unselected expert (the winners are
    // taken out first: the packed rounds leave ko as it was)
    const float last_lo = readlane_f32(win.y, K - 1);
    const int last_e = __builtin_amdgcn_readlane(r.e, K - 1);
    bool out[4];
#pragma unroll
    for (int j = 0; j < 4; j++) out[j] = ko[j] != 0u;
    for (int k = 0; k < K; k++) {
      const int ew = __builtin_amdgcn_readlane(r.e, k);
#pragma unroll
      for (int j = 0; j < 4; j++) out[j] = out[j] && lane + 64 * j != ew;
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int ee = lane + 64 * j;
      if (ee < E && out[j] && !(last_lo > kh[j] || (last_lo == kh[j] && last_e < ee))) ok = false;
    }
    if (__any(!ok)) {
      float floor = lane < K ? win.y : __builtin_huge_valf();
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) floor = fminf(floor, __shfl_xor(floor, off));
      // outputs of their own, live only on this path (the common path then
      // keeps nothing in the stack slots the call needs)
      int ex;
      float sx;
      select_exact(kb, E, K, floor, src, status, report, ex, sx);
      r = SelIds{ex, sx, true};
    }
  }
  return r;
}

__device__ inline float select_gate(const float4* kb, int K, float scale, const SelIds& r) {
  const int lane = threadIdx.x & 63;
  const float s = r.exact ? r.s : (lane < K ? kb[r.e].w : 0.0f);
  double ssum = 0.0;
  for (int k = 0; k < K; k++) ssum += (double)readlane_f32(s, k);
  return lane < K ? (float)((double)scale * (double)s / ssum) : 0.0f;
}

// Selection kernel.  Grid T, one wave per token: reads the key intervals
// written by k_route_score (visible at the kernel boundary), picks the top K
// and writes ids and gates.
// Grid (T) of one wave each; with a.items one workgroup of T waves (wave t:
// token t), whose ids meet in LDS for the item list.
__global__ __launch_bounds__(1024) void k_route_select(RouteArgs a) {
  __shared__ int s_e[kSelItemsMax], s_sorted[kSelItemsMax];
  const int lane = threadIdx.x & 63;
  const int t = a.items ? (int)(threadIdx.x >> 6) : (int)blockIdx.x;
  int e;
  float w;
  // the router input of token t: the normalised row when the scoring wrote it
  RouteSrc src;
  if (a.norm_w) {
    src.x = a.xn_out + (size_t)t * a.H;
    src.x_dt = DS4MOE_BF16;
  } else {
    src.x = (const char*)a.x + (size_t)t * a.H * (a.x_dt == DS4MOE_F32 ? 4 : 2);
    src.x_dt = a.x_dt;
  }
  src.W = a.W;
  src.w_dt = a.w_dt;
  src.bias = a.bias;
  src.H = a.H;
  const SelIds sel = select_ids(a.kbuf + (size_t)t * a.E, a.E, a.K, a.status, true, src);
  e = lane < a.K ? sel.e : 0;
  w = select_gate(a.kbuf + (size_t)t * a.E, a.K, a.scale, sel);
  if (lane < a.K) {
    a.ids[(size_t)t * a.K + lane] = e;
    a.wts[(size_t)t * a.K + lane] = w;
    if (a.items) s_e[t * a.K + lane] = e;
  }
  if (!a.items) return;
  __syncthreads();
  const int n = a.T * a.K;
  // rank of pair p in the order (expert, p), one thread per pair
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    const int ep = s_e[p];
    int r = 0;
    for (int q = 0; q < n; q++) r += (s_e[q] < ep || (s_e[q] == ep && q < p)) ? 1 : 0;
    a.perm[r] = p;
    s_sorted[r] = ep;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // an item starts wherever the expert changes; its index counts the starts before it
  bool st[kSelItemsMax / 64];
  uint64_t m[kSelItemsMax / 64];
#pragma unroll
  for (int h = 0; h < kSelItemsMax / 64; h++) {
    const int i = 64 * h + lane;
    st[h] = i < n && (i == 0 || s_sorted[i] != s_sorted[i - 1]);
    m[h] = __ballot(st[h]);
  }
  int before = 0;
#pragma unroll
  for (int h = 0; h < kSelItemsMax / 64; h++) {
    const int i = 64 * h + lane;
    const int u = before + __popcll(m[h] & ((1ull << lane) - 1ull));
    if (st[h]) {
      int c = 1;
      while (i + c < n && s_sorted[i + c] == s_sorted[i]) c++;
      a.items[3 * u] = s_sorted[i];
      a.items[3 * u + 1] = i;
      a.items[3 * u + 2] = c;
    }
    before += __popcll(m[h]);
  }
  if (lane == 0) {
    a.n_items[0] = before;
    a.n_items[1] = before;
  }
}

// Hash routing of token t: its row of the table.  An invalid token id or
// table row raises a fault bit and routes to experts 0..K-1 so that later
// kernels stay in bounds.
__device__ inline void route_hash_token(int t, const int32_t* tok, const int32_t* table, int vocab,
                                        int E, int K, float scale, int32_t* ids, float* wts,
                                        uint32_t* status) {
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

// Hash routing: one thread per token.
__global__ void k_route_hash(const int32_t* tok, const int32_t* table, int vocab, int E, int K, int T,
                             float scale, int32_t* ids, float* wts, uint32_t* status) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  route_hash_token(t, tok, table, vocab, E, K, scale, ids, wts, status);
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

__device__ void make_items_wave(const int32_t* counts, const int32_t* offsets, int E, int TK, int T,
                                int with_shared, int32_t* items, int32_t* n_items);

// Counting sort of the pairs by expert (stable: pair order within an
// expert), one workgroup.  With items (nullable) the work list of the
// grouped kernels is built too (make_items_wave, wave 1, from the counts and
// offsets in LDS while wave 0 scatters).
__global__ __launch_bounds__(1024) void k_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                                  int32_t* offsets, int32_t* perm, int32_t* inv,
                                                  uint32_t* status, int T, int with_shared,
                                                  int32_t* items, int32_t* n_items) {
  __shared__ int tab[kPermChunks * 256];  // [chunk][expert]: counts, then first positions
  __shared__ uint8_t eid[kPermMax];
  __shared__ int base[257], s_cnt[256];
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
  if (tid < 64) {  // exclusive scan over the experts: four per lane, then over the lanes
    int c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = 4 * tid + j;
      c[j] = e < E ? base[e] : 0;
      sum += c[j];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d);
      if (tid >= d) incl += u;
    }
    int run = incl - sum;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = 4 * tid + j;
      if (e < E) {
        counts[e] = c[j];
        offsets[e] = run;
        s_cnt[e] = c[j];
        base[e] = run;
      }
      run += c[j];
    }
    if (tid == 63) offsets[E] = run;
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
  } else if (items && tid < 2 * 64) {
    make_items_wave(s_cnt, base, E, n, T, with_shared, items, n_items);
  }
}

}  // namespace ds4
