// ffn_shared.hip -- the shared expert (Q8_0 gate, up and down with the
// V4-Flash expert shape) in few-token calls: per-token matvecs (one grid row
// per token) and read-once variants for a few tokens per grid row.  In layer
// calls of up to ten tokens the gate/up blocks run inside the router's
// scoring launch (k_route_score_shared); otherwise they follow the routed
// kernels.  Up to four tokens (Q2_K routed down) the down runs as a seventh
// slot of the routed batch-1 down, else as a kernel of its own.
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, section
// "MoE FFN 部の中身" (an always-on shared expert whose output is added to
// the routed weighted sum, unscaled).  Format: Q8_0, 34 bytes per 32 values
// (fp16 d, then 32 int8 codes; y = d c), FLOW quantisation table.
//
// A lane covers 64 consecutive values of a row: two Q8_0 blocks, i.e. the 68
// bytes at byte 68L of the row (4-byte aligned), read as 17 dwords.  Its
// activations are held as 16-bit fixed point with one scale (q4k_fix: the
// 16-bit pairs (4k, 4k+2) and (4k+1, 4k+3) of each half), and a code dword
// XOR 0x80808080 holds the codes plus 128 as unsigned bytes, so the masks
// 0x00FF00FF on it and on it shifted by 8 put them into 16-bit lanes in the
// same pairs: v_dot2_i32_i16 multiplies them exactly, and 128 times the
// half's fixed-point sum is taken off again.  Each block's d is applied once.
#include "dev_common.h"

namespace ds4 {

constexpr int kShRowGu = kH / 32 * kQ80Bytes;  // 4352 bytes per gate/up row
constexpr int kShRowDn = kI / 32 * kQ80Bytes;  // 2176 bytes per down row

struct SharedB1Args {
  const uint16_t* x;                 // [T][4096] bf16
  const uint8_t *gate, *up, *down;   // Q8_0: [2048][4352 B], [2048][4352 B], [4096][2176 B]
  float* h;                          // [T][2048] fp32 SwiGLU rows (workspace)
  float* out;                        // [T][4096]: out (or the residual) += shared output
  uint32_t* status;
};

__device__ inline void q80_pair_load(const uint8_t* p, uint32_t (&D)[17]) {
  const uint32_t* q = (const uint32_t*)p;
#pragma unroll
  for (int j = 0; j < 17; j++) D[j] = q[j];
}

// Partial dot product of a lane's 64 values with its fixed-point activations
// (before the lane's scale).  Block 0: d in bytes 0-1, codes in 2..33 (each
// code dword straddles two loaded dwords); block 1: d in bytes 34-35, codes
// in 36..67 (dwords 9..16).
__device__ inline float q80_dot64(const uint32_t (&D)[17], const uint32_t* xl, const uint32_t* xh,
                                  int sl, int sh) {
  int a0 = 0, a1 = 0;  // |a| < 32 * 255 * 32767 < 2^31
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const uint32_t w0 = align_bytes(D[k + 1], D[k], 2) ^ 0x80808080u;
    const uint32_t w1 = D[9 + k] ^ 0x80808080u;
    a0 = sdot2(w0 & 0x00FF00FFu, xl[2 * k], a0);
    a0 = sdot2((w0 >> 8) & 0x00FF00FFu, xl[2 * k + 1], a0);
    a1 = sdot2(w1 & 0x00FF00FFu, xh[2 * k], a1);
    a1 = sdot2((w1 >> 8) & 0x00FF00FFu, xh[2 * k + 1], a1);
  }
  const float d0 = f16_bits_to_f32(D[0] & 0xFFFFu), d1 = f16_bits_to_f32(D[8] >> 16);
  return d0 * (float)(a0 - 128 * sl) + d1 * (float)(a1 - 128 * sh);
}

// gate/up + SwiGLU of the shared expert.  Grid (2048 / 8, T), 256 threads:
// wave w of block b handles features 8b + 2w and 8b + 2w + 1 (their gate and
// up rows) for token blockIdx.y.  The weights are requested right behind the
// token's activations, before the fixed-point conversion (or, with the
// normalised input, right behind the RMSNorm's loads: shared_gateup_b1_rows
// first, shared_gateup_b1_block on the rows afterwards).
// xrow: the token's input row (a.x + t * 4096, or a copy in LDS)
__device__ inline void shared_gateup_b1_rows(const SharedB1Args& a, int bx, uint32_t (&D)[4][17]) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int f0 = 8 * bx + 2 * w;
#pragma unroll
  for (int r = 0; r < 4; r++) {  // gate f0, gate f0+1, up f0, up f0+1
    const uint8_t* base = (r < 2 ? a.gate : a.up) + (size_t)(f0 + (r & 1)) * kShRowGu;
    q80_pair_load(base + 68 * lane, D[r]);
  }
}
template <bool ROWS_GIVEN = false>
__device__ inline void shared_gateup_b1_block(const SharedB1Args& a, int bx, int t,
                                              const uint16_t* xrow, uint32_t (*Dg)[17] = nullptr) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int f0 = 8 * bx + 2 * w;
  const uint4* xp = (const uint4*)(xrow + 64 * lane);
  uint4 xq[8];
#pragma unroll
  for (int q = 0; q < 8; q++) xq[q] = xp[q];
  uint32_t Dl[4][17];
  if constexpr (!ROWS_GIVEN) shared_gateup_b1_rows(a, bx, Dl);
  uint32_t (*D)[17] = ROWS_GIVEN ? Dg : Dl;
  // keep every load ahead of the conversion (the scheduler would otherwise
  // issue the weights only after the activations have returned)
  __builtin_amdgcn_sched_barrier(0);
  auto xval = [&](int i) {
    const uint4 q = xq[i >> 3];
    const uint32_t ww = (i & 6) == 0 ? q.x : (i & 6) == 2 ? q.y : (i & 6) == 4 ? q.z : q.w;
    return bf16_bits_to_f32((i & 1) ? (ww >> 16) : (ww & 0xFFFFu));
  };
  uint32_t xl[16], xh[16];
  int sl, sh;
  const float S = q4k_fix(xval, xl, xh, sl, sh);
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; r++) v[r] = wave_sum(S * q80_dot64(D[r], xl, xh, sl, sh));
  if (lane < 2) {
    const float g = lane ? v[1] : v[0], u = lane ? v[3] : v[2];
    a.h[(size_t)t * kI + f0 + lane] = silu(g) * u;
  }
}
__global__ __launch_bounds__(256) void k_shared_gateup_q80_b1(SharedB1Args a) {
  shared_gateup_b1_block(a, blockIdx.x, blockIdx.y, a.x + (size_t)blockIdx.y * kH);
}

// down of the shared expert, added to the output.  Grid (4096 / 16, T), 256
// threads: wave w of block b handles rows 16b + 4w .. +3, two at a time (wave
// half u takes rows +u and +2+u); lane L of a half covers columns 64L .. +63.
__global__ __launch_bounds__(256) void k_shared_down_q80_b1(SharedB1Args a) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = lane >> 5, L = lane & 31;
  const int t = blockIdx.y;
  const int r0 = 16 * blockIdx.x + 4 * w;
  const float4* hp = (const float4*)(a.h + (size_t)t * kI + 64 * L);
  float4 hv[16];
#pragma unroll
  for (int q = 0; q < 16; q++) hv[q] = hp[q];
  uint32_t D0[17], D1[17];
  q80_pair_load(a.down + (size_t)(r0 + u) * kShRowDn + 68 * L, D0);
  q80_pair_load(a.down + (size_t)(r0 + 2 + u) * kShRowDn + 68 * L, D1);
  __builtin_amdgcn_sched_barrier(0);  // all loads ahead of the conversion
  auto hval = [&](int i) {
    const float4 q = hv[i >> 2];
    return (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
  };
  uint32_t xl[16], xh[16];
  int sl, sh;
  const float S = q4k_fix(hval, xl, xh, sl, sh);
  float p0 = S * q80_dot64(D0, xl, xh, sl, sh), p1 = S * q80_dot64(D1, xl, xh, sl, sh);
  // sums over each wave half: DPP inside rows of 16, then rows 0 + 1 and 2 + 3
  p0 += dpp_f32<0xB1>(p0);
  p0 += dpp_f32<0x4E>(p0);
  p0 += dpp_f32<0x141>(p0);
  p0 += dpp_f32<0x140>(p0);
  p1 += dpp_f32<0xB1>(p1);
  p1 += dpp_f32<0x4E>(p1);
  p1 += dpp_f32<0x141>(p1);
  p1 += dpp_f32<0x140>(p1);
  auto rl = [](float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  };
  const float t0 = rl(p0, 0) + rl(p0, 16), t1 = rl(p0, 32) + rl(p0, 48);  // rows r0, r0 + 1
  const float t2 = rl(p1, 0) + rl(p1, 16), t3 = rl(p1, 32) + rl(p1, 48);  // rows r0 + 2, r0 + 3
  if (lane < 4) {
    const float tot = lane == 0 ? t0 : lane == 1 ? t1 : lane == 2 ? t2 : t3;
    a.out[(size_t)t * kH + r0 + lane] += tot;
  }
}

// The same two matvecs for a few tokens at once: grid row y takes tokens
// kShFewTok y .. +kShFewTok-1 (of T).  Every wave requests its weight rows
// once; then wave w turns token w's activations into the lanes' 16-bit
// fixed-point form (q4k_fix: the same for every wave, since lane L covers
// the same 64 columns in each) and leaves it in LDS, and every wave runs
// through the tokens' dot products from there.  A lane's record is 36 words
// (xl[16], xh[16], sl, sh, S, one spare): at that stride the 16 lanes one
// 16-byte read serves hit 16 distinct bank groups.
constexpr int kShFewTok = 4;   // tokens per grid row: one per wave
constexpr int kShFx = 36;      // words of a lane's fixed-point record

__device__ inline void fx_store(uint32_t* r, const uint32_t* xl, const uint32_t* xh, int sl, int sh,
                                float S) {
#pragma unroll
  for (int q = 0; q < 16; q += 4) {
    *(uint4*)(r + q) = make_uint4(xl[q], xl[q + 1], xl[q + 2], xl[q + 3]);
    *(uint4*)(r + 16 + q) = make_uint4(xh[q], xh[q + 1], xh[q + 2], xh[q + 3]);
  }
  *(uint4*)(r + 32) = make_uint4((uint32_t)sl, (uint32_t)sh, __float_as_uint(S), 0u);
}

__device__ inline float fx_load(const uint32_t* r, uint32_t* xl, uint32_t* xh, int& sl, int& sh) {
#pragma unroll
  for (int q = 0; q < 16; q += 4) {
    const uint4 a = *(const uint4*)(r + q), b = *(const uint4*)(r + 16 + q);
    xl[q] = a.x; xl[q + 1] = a.y; xl[q + 2] = a.z; xl[q + 3] = a.w;
    xh[q] = b.x; xh[q + 1] = b.y; xh[q + 2] = b.z; xh[q + 3] = b.w;
  }
  const uint4 c = *(const uint4*)(r + 32);
  sl = (int)c.x;
  sh = (int)c.y;
  return __uint_as_float(c.z);
}

// gate/up: grid (2048 / 8, rows of kShFewTok tokens), 256 threads, rows as in
// k_shared_gateup_q80_b1.
__device__ inline void shared_gateup_few_block(const SharedB1Args& a, int T, int bx, int by) {
  __shared__ uint32_t fx[kShFewTok * 64 * kShFx];
  const int t0 = kShFewTok * by, nt = min(kShFewTok, T - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f0 = 8 * bx + 2 * w;
  uint32_t D[4][17];  // gate f0, gate f0+1, up f0, up f0+1
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const uint8_t* base = (r < 2 ? a.gate : a.up) + (size_t)(f0 + (r & 1)) * kShRowGu;
    q80_pair_load(base + 68 * lane, D[r]);
  }
  if (w < nt) {  // wave w converts token t0 + w
    const uint4* xp = (const uint4*)(a.x + (size_t)(t0 + w) * kH + 64 * lane);
    uint4 xq[8];
#pragma unroll
    for (int q = 0; q < 8; q++) xq[q] = xp[q];
    auto xval = [&](int i) {
      const uint4 q = xq[i >> 3];
      const uint32_t ww = (i & 6) == 0 ? q.x : (i & 6) == 2 ? q.y : (i & 6) == 4 ? q.z : q.w;
      return bf16_bits_to_f32((i & 1) ? (ww >> 16) : (ww & 0xFFFFu));
    };
    uint32_t xl[16], xh[16];
    int sl, sh;
    const float S = q4k_fix(xval, xl, xh, sl, sh);
    fx_store(fx + (w * 64 + lane) * kShFx, xl, xh, sl, sh, S);
  }
  __syncthreads();
  for (int t = 0; t < nt; t++) {
    uint32_t xl[16], xh[16];
    int sl, sh;
    const float S = fx_load(fx + (t * 64 + lane) * kShFx, xl, xh, sl, sh);
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; r++) v[r] = wave_sum(S * q80_dot64(D[r], xl, xh, sl, sh));
    if (lane < 2) {
      const float g = lane ? v[1] : v[0], u = lane ? v[3] : v[2];
      a.h[(size_t)(t0 + t) * kI + f0 + lane] = silu(g) * u;
    }
  }
}
__global__ __launch_bounds__(256) void k_shared_gateup_q80_few(SharedB1Args a, int T) {
  shared_gateup_few_block(a, T, blockIdx.x, blockIdx.y);
}

// The router's scoring and the shared expert's gate/up in one launch: the
// shared expert does not depend on the routing, so its weight stream runs
// beside the scoring, whose blocks wait mostly on memory latency.  Grid
// (E + 2048 / 8, T), 256 threads: blocks x < E score expert x for token y
// (k_route_score<NORM, VEC>); the others are the shared gate/up blocks
// x - E (per token, or FEW: for the tokens of grid row y of kShFewTok).
// NORM (VEC, per token): the input is RMSNorm(residual), which the scoring
// blocks compute and block 0 stores; a shared block cannot wait for that
// store, so it computes the normalised row itself with the scoring's own
// code and order of operations (the same bits) into LDS.
template <bool VEC, bool FEW, bool NORM>
__global__ __launch_bounds__(256) void k_route_score_shared(RouteArgs r, SharedB1Args s, int T) {
  static_assert(!NORM || (VEC && !FEW), "normalised input: per-token shared blocks only");
  if ((int)blockIdx.x < r.E) {
    route_score_block<NORM, VEC>(r, blockIdx.x, blockIdx.y);
  } else if (NORM) {
    __shared__ double shd[8];
    __shared__ uint4 xs4[kH / 8];
    uint16_t* xs = (uint16_t*)xs4;
    // the RMSNorm's loads, then the weight rows, then the norm: its waits
    // (the vector memory counter retires in order) do not wait for weights
    float rr[2][8], nw[2][8];
    rms_load_vec(r, blockIdx.y, rr, nw);
    uint32_t D[4][17];
    shared_gateup_b1_rows(s, blockIdx.x - r.E, D);
    __builtin_amdgcn_sched_barrier(0);
    const double ns = rms_scale_of(r, shd, rr);
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int u = 0; u < 8; u++)
        xs[2048 * j + 8 * threadIdx.x + u] =
            (uint16_t)f64_to_bf16_bits((double)rr[j][u] * ns * (double)nw[j][u]);
    __syncthreads();
    shared_gateup_b1_block<true>(s, blockIdx.x - r.E, blockIdx.y, xs, D);
  } else if (FEW) {
    if ((int)blockIdx.y * kShFewTok < T) shared_gateup_few_block(s, T, blockIdx.x - r.E, blockIdx.y);
  } else {
    shared_gateup_b1_block(s, blockIdx.x - r.E, blockIdx.y, s.x + (size_t)blockIdx.y * kH);
  }
}

// down: grid (4096 / 16, rows of kShFewTok tokens), 256 threads, rows as in
// k_shared_down_q80_b1 (both wave halves cover the same 64 columns per lane,
// so the lower half converts); out[t] (or the residual) += the shared output.
__global__ __launch_bounds__(256) void k_shared_down_q80_few(SharedB1Args a, int T) {
  __shared__ uint32_t fx[kShFewTok * 32 * kShFx];
  const int t0 = kShFewTok * blockIdx.y, nt = min(kShFewTok, T - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = lane >> 5, L = lane & 31;
  const int r0 = 16 * blockIdx.x + 4 * w;
  uint32_t D0[17], D1[17];
  q80_pair_load(a.down + (size_t)(r0 + u) * kShRowDn + 68 * L, D0);
  q80_pair_load(a.down + (size_t)(r0 + 2 + u) * kShRowDn + 68 * L, D1);
  if (w < nt) {  // wave w converts token t0 + w
    const float4* hp = (const float4*)(a.h + (size_t)(t0 + w) * kI + 64 * L);
    float4 hv[16];
#pragma unroll
    for (int q = 0; q < 16; q++) hv[q] = hp[q];
    auto hval = [&](int i) {
      const float4 q = hv[i >> 2];
      return (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
    };
    uint32_t xl[16], xh[16];
    int sl, sh;
    const float S = q4k_fix(hval, xl, xh, sl, sh);
    if (u == 0) fx_store(fx + (w * 32 + L) * kShFx, xl, xh, sl, sh, S);
  }
  __syncthreads();
  auto rl = [](float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  };
  for (int t = 0; t < nt; t++) {
    uint32_t xl[16], xh[16];
    int sl, sh;
    const float S = fx_load(fx + (t * 32 + L) * kShFx, xl, xh, sl, sh);
    float p0 = S * q80_dot64(D0, xl, xh, sl, sh), p1 = S * q80_dot64(D1, xl, xh, sl, sh);
    p0 += dpp_f32<0xB1>(p0);
    p0 += dpp_f32<0x4E>(p0);
    p0 += dpp_f32<0x141>(p0);
    p0 += dpp_f32<0x140>(p0);
    p1 += dpp_f32<0xB1>(p1);
    p1 += dpp_f32<0x4E>(p1);
    p1 += dpp_f32<0x141>(p1);
    p1 += dpp_f32<0x140>(p1);
    const float s0 = rl(p0, 0) + rl(p0, 16), s1 = rl(p0, 32) + rl(p0, 48);  // rows r0, r0 + 1
    const float s2 = rl(p1, 0) + rl(p1, 16), s3 = rl(p1, 32) + rl(p1, 48);  // rows r0 + 2, r0 + 3
    if (lane < 4) {
      const float tot = lane == 0 ? s0 : lane == 1 ? s1 : lane == 2 ? s2 : s3;
      a.out[(size_t)(t0 + t) * kH + r0 + lane] += tot;
    }
  }
}

// The shared expert's down as the seventh slot of k_down_q2k_b1<true, false>: rows
// row0 + 2m + u (m < 4) of the wave, lane L of half u covering columns
// 64L .. +63 (two Q8_0 blocks) of the shared SwiGLU row sh_h (global memory);
// the row's values and the first two steps' weights are requested before the
// values are converted, the last two steps' weights right after.
__device__ void shared_down_slot(const float4* sh_h, const uint8_t* sh_down, int row0, int lane,
                                 float* pr) {
  const int u = lane >> 5, L = lane & 31;
  float4 hv[16];
#pragma unroll
  for (int q = 0; q < 16; q++) hv[q] = sh_h[16 * L + q];
  uint32_t D0[17], D1[17];
  q80_pair_load(sh_down + (size_t)(row0 + u) * kShRowDn + 68 * L, D0);
  q80_pair_load(sh_down + (size_t)(row0 + 2 + u) * kShRowDn + 68 * L, D1);
  auto hval = [&](int i) {
    const float4 q = hv[i >> 2];
    return (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
  };
  uint32_t xl[16], xh[16];
  int sl, sh;
  const float S = q4k_fix(hval, xl, xh, sl, sh);
  uint32_t D2[17], D3[17];
  q80_pair_load(sh_down + (size_t)(row0 + 4 + u) * kShRowDn + 68 * L, D2);
  q80_pair_load(sh_down + (size_t)(row0 + 6 + u) * kShRowDn + 68 * L, D3);
  pr[0] = S * q80_dot64(D0, xl, xh, sl, sh);
  pr[1] = S * q80_dot64(D1, xl, xh, sl, sh);
  pr[2] = S * q80_dot64(D2, xl, xh, sl, sh);
  pr[3] = S * q80_dot64(D3, xl, xh, sl, sh);
}

// The few-token shared-expert kernels apply: Q8_0 gate, up and down of the
// V4-Flash shape, bf16 activations, 4-byte-aligned weights.
inline bool shared_b1_ok(const ds4moe_shape& s, const ds4moe_experts& sh, const void* x,
                         int32_t x_dt) {
  return sh.gate_qtype == DS4MOE_Q8_0 && sh.up_qtype == DS4MOE_Q8_0 &&
         sh.down_qtype == DS4MOE_Q8_0 && sh.inter == kI && s.hidden == kH &&
         x_dt == DS4MOE_BF16 && ((uintptr_t)x % 16) == 0 &&
         (((uintptr_t)sh.gate | (uintptr_t)sh.up | (uintptr_t)sh.down) % 4) == 0;
}

}  // namespace ds4
