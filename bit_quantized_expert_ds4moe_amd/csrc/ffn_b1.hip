// ffn_b1.hip -- batch-1 decode matvecs for the V4-Flash expert shape
// (hidden 4096, intermediate 2048, IQ2_XXS gate/up, Q2_K down), gfx950.
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, section
// "MoE FFN 部の中身": E(x) = W_down (SiLU(W_gate x) * W_up x), y = sum_k g_k E_k.
// Formats: DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec,
// sections 3 (Q2_K, 84 B / 256) and 4 (IQ2_XXS, 66 B / 256).
//
// At batch 1 every weight byte is used once, so these kernels stream HBM and
// the work per weight value must stay near one VALU op.  Design:
//  * A wave owns a row; lane l always covers the same 64 (gate/up) or 32
//    (down) columns, so its slice of the activation lives in registers for
//    the whole kernel and only weights move.
//  * gate/up: an IQ2_XXS grid entry becomes four bf16 pairs from a 4 KB LDS
//    table, a 7-bit sign mask (with its even-parity eighth bit) becomes four
//    XOR masks from a 2 KB LDS table, and v_dot2_f32_bf16 multiplies them with
//    the bf16 activation.  Grid values (< 128) are exact in bf16, so the dot
//    products are exact and only the fp32 accumulation rounds.  The group
//    scale d*(2s+1)/8 multiplies the 32-value partial sum once.
//  * down: the SwiGLU output h is rounded to binary16 (prescaled by 4^-s for
//    the bit pair it meets) once per call; a Q2_K code is masked in place
//    inside a 16-bit lane so that the masked bits, read as a binary16
//    subnormal, equal 4^s q 2^-24, and v_dot2_f32_f16 does two products per
//    op with no offset to remove.  Scales, mins, 2^24 and the gate weight are
//    applied once per 8 values.  The min term uses the sum of the same binary16
//    h values, so the result is exactly the dot product of the dequantised row
//    with the binary16-rounded h, accumulated in fp32.
//  * Row reductions use DPP inside rows of 16 lanes and four readlanes.
#include "dev_common.h"

namespace ds4 {

constexpr int kH = 4096;        // hidden size of the fast path
constexpr int kI = 2048;        // intermediate size of the fast path
constexpr int kRowIq2 = 16 * kIq2Bytes;  // 1056 bytes per gate/up row
constexpr int kRowQ2k = 8 * kQ2kBytes;   // 672 bytes per down row

// Layout of the binary16 SwiGLU output consumed by the down matvec, per
// routed slot: [64 lanes][16 dwords]; dword 4s+m of lane 8b+4hh+c holds the
// values i, i+1 with i = 256b + 128hh + 32s + 8c + 2m, scaled by 4^-s.
__device__ inline int hs_half_index(int k, int i) {
  int b = i >> 8, v = i & 255, hh = v >> 7, s = (v >> 5) & 3, lp = v & 31, c = lp >> 3, u = lp & 7;
  int lane = 8 * b + 4 * hh + c;
  return (((k * 64 + lane) * 16) + 4 * s + (u >> 1)) * 2 + (u & 1);
}

__device__ inline void store_h16(uint16_t* hs, int k, int i, float hv, uint32_t* status) {
  int s = (i >> 5) & 3;
  float scaled = hv * (s == 0 ? 1.0f : s == 1 ? 0.25f : s == 2 ? 0.0625f : 0.015625f);
  if (!(fabsf(scaled) <= 65504.0f)) raise_fault(status, DS4MOE_FAULT_F16_RANGE);
  hs[hs_half_index(k, i)] = (uint16_t)f32_to_f16_bits(scaled);
}

// LDS tables: grid entry -> 4 bf16 pairs; 7-bit sign mask -> 4 XOR masks.
__device__ inline void build_iq2_tables(const uint8_t* grid, uint4* gt, uint4* mt) {
  int t = threadIdx.x;
  if (t < 256) {
    const uint8_t* g = grid + 8 * t;
    uint32_t w[4];
    for (int m = 0; m < 4; m++) {
      uint32_t lo = __float_as_uint((float)g[2 * m]) >> 16;
      uint32_t hi = __float_as_uint((float)g[2 * m + 1]) >> 16;
      w[m] = lo | (hi << 16);
    }
    gt[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (t < 128) {
    uint32_t s8 = (uint32_t)t | ((uint32_t)(__popc(t) & 1) << 7);
    uint32_t w[4];
    for (int m = 0; m < 4; m++)
      w[m] = (((s8 >> (2 * m)) & 1u) << 15) | (((s8 >> (2 * m + 1)) & 1u) << 31);
    mt[t] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One IQ2_XXS row segment: lane covers block b = lane/4, groups 2j, 2j+1
// (j = lane%4), i.e. 64 columns starting at 256b + 64j.  Returns the lane's
// partial dot product with the register-resident activation xr.
__device__ inline float iq2_row_partial(const uint8_t* row, int lane, const uint32_t* xr,
                                        const uint4* gt, const uint4* mt) {
  const int b = lane >> 2, j = lane & 3;
  const uint8_t* blk = row + b * kIq2Bytes;
  // fp16 block scale d (2-byte aligned field)
  uintptr_t da = (uintptr_t)blk;
  uint32_t dw = *(const uint32_t*)(da & ~(uintptr_t)3);
  float d = f16_bits_to_f32((da & 2) ? (dw >> 16) : (dw & 0xFFFFu));
  // 16 bytes of group data at blk + 2 + 16j, 2- or 4-byte aligned
  uintptr_t ga = (uintptr_t)(blk + 2 + 16 * j);
  uint32_t sh = (uint32_t)(ga & 3);
  const uint32_t* gp = (const uint32_t*)(ga - sh);
  uint32_t w0 = gp[0], w1 = gp[1], w2 = gp[2], w3 = gp[3];
  // tail bytes: only needed when misaligned; the address stays inside the group
  uint32_t w4 = *(const uint16_t*)(ga - sh + (sh ? 16 : 14));
  uint32_t g[4];
  g[0] = align_bytes(w1, w0, sh);
  g[1] = align_bytes(w2, w1, sh);
  g[2] = align_bytes(w3, w2, sh);
  g[3] = align_bytes(w4, w3, sh);
  float acc = 0.0f;
#pragma unroll
  for (int grp = 0; grp < 2; grp++) {
    uint32_t idxw = g[2 * grp], sw = g[2 * grp + 1];
    float dg = d * (float)(2u * (sw >> 28) + 1u) * 0.125f;
    float gacc = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      uint4 gv = gt[(idxw >> (8 * kk)) & 0xFFu];
      uint4 mv = mt[(sw >> (7 * kk)) & 0x7Fu];
      const uint32_t* xp = xr + grp * 16 + kk * 4;
      gacc = dot2_bf16(gv.x ^ mv.x, xp[0], gacc);
      gacc = dot2_bf16(gv.y ^ mv.y, xp[1], gacc);
      gacc = dot2_bf16(gv.z ^ mv.z, xp[2], gacc);
      gacc = dot2_bf16(gv.w ^ mv.w, xp[3], gacc);
    }
    acc = fmaf(dg, gacc, acc);
  }
  return acc;
}

// gate/up + SwiGLU for one token.  Grid (I / (4*ROWS), K), 256 threads.
template <int ROWS>
__global__ __launch_bounds__(256) void k_gateup_iq2_b1(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ gate,
                                                       const uint8_t* __restrict__ up,
                                                       const uint8_t* __restrict__ grid,
                                                       const int32_t* __restrict__ ids, int E,
                                                       uint16_t* __restrict__ hs,
                                                       uint32_t* status) {
  __shared__ uint4 gt[256];
  __shared__ uint4 mt[128];
  build_iq2_tables(grid, gt, mt);
  const int k = blockIdx.y;
  int e = ids[k];
  if (e < 0 || e >= E) {
    if (threadIdx.x == 0 && blockIdx.x == 0) raise_fault(status, DS4MOE_FAULT_BAD_ID);
    e = 0;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = lane >> 2, j = lane & 3;
  uint32_t xr[32];
  const uint4* xp = (const uint4*)(x + 256 * b + 64 * j);
#pragma unroll
  for (int q = 0; q < 8; q++) {
    uint4 v = xp[q];
    xr[4 * q] = v.x;
    xr[4 * q + 1] = v.y;
    xr[4 * q + 2] = v.z;
    xr[4 * q + 3] = v.w;
  }
  __syncthreads();
  const size_t ebase = (size_t)e * kI;
#pragma unroll 1
  for (int r = 0; r < ROWS; r++) {
    const int i = (blockIdx.x * 4 + wave) * ROWS + r;
    float pg = iq2_row_partial(gate + (ebase + i) * kRowIq2, lane, xr, gt, mt);
    float pu = iq2_row_partial(up + (ebase + i) * kRowIq2, lane, xr, gt, mt);
    float g = wave_sum(pg), u = wave_sum(pu);
    if (lane == 0) store_h16(hs, k, i, silu(g) * u, status);
  }
}

// down + weighted combine (+ residual) for one token.  Grid H/(4*ROWS),
// 256 threads; K = 6 routed slots.
template <int ROWS, int K>
__global__ __launch_bounds__(256) void k_down_q2k_b1(const uint16_t* __restrict__ hs,
                                                     const uint8_t* __restrict__ down,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ wts, int E,
                                                     float* __restrict__ out,
                                                     float* __restrict__ residual,
                                                     uint32_t* status) {
  __shared__ uint4 hl[K * 64 * 4];
  {
    const uint4* src = (const uint4*)hs;
    for (int q = threadIdx.x; q < K * 64 * 4; q += 256) hl[q] = src[q];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = lane >> 3, q8 = lane & 7, hh = q8 >> 2, c = q8 & 3;
  int ek[K];
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; k++) {
    int e = ids[k];
    if (e < 0 || e >= E) {
      if (threadIdx.x == 0 && blockIdx.x == 0) raise_fault(status, DS4MOE_FAULT_BAD_ID);
      e = 0;
    }
    ek[k] = e;
    wk[k] = wts[k] * 16777216.0f;  // folds the 2^24 of the binary16 subnormal codes
  }
  __syncthreads();
  uint32_t hr[K][16];
  uint32_t xs[K][2];
  const uint32_t ONES = 0x3C003C00u;  // binary16 pair (1, 1)
#pragma unroll
  for (int k = 0; k < K; k++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      uint4 v = hl[(k * 64 + lane) * 4 + q];
      hr[k][4 * q] = v.x;
      hr[k][4 * q + 1] = v.y;
      hr[k][4 * q + 2] = v.z;
      hr[k][4 * q + 3] = v.w;
    }
    // X_s = sum of the 8 binary16 values of bit pair s (undo 4^-s), / 16 for
    // the min nibble read as 16*m.
    float X[4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
      float t = dot2_f16(hr[k][4 * s], ONES, 0.0f);
      t = dot2_f16(hr[k][4 * s + 1], ONES, t);
      t = dot2_f16(hr[k][4 * s + 2], ONES, t);
      t = dot2_f16(hr[k][4 * s + 3], ONES, t);
      X[s] = t * (float)(1 << (2 * s)) * 0.0625f;
    }
    xs[k][0] = f32_to_f16_bits(X[0]) | (f32_to_f16_bits(X[1]) << 16);
    xs[k][1] = f32_to_f16_bits(X[2]) | (f32_to_f16_bits(X[3]) << 16);
  }
  // byte selectors: scale bytes (c/2) + {0,2,4,6} of the 8-byte window
  const uint32_t cb = (uint32_t)(c >> 1);
  const uint32_t ssel = cb | ((cb + 2) << 8) | ((cb + 4) << 16) | ((cb + 6) << 24);
  const int qoff = 16 + 32 * hh + 8 * c, soff = 8 * hh;
#pragma unroll 1
  for (int r = 0; r < ROWS; r++) {
    const int row = (blockIdx.x * 4 + wave) * ROWS + r;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < K; k++) {
      const uint8_t* blk = down + ((size_t)ek[k] * kH + row) * kRowQ2k + b * kQ2kBytes;
      uint2 qv = *(const uint2*)(blk + qoff);
      uint2 sv = *(const uint2*)(blk + soff);
      uint32_t dd = *(const uint32_t*)(blk + 80);
      // 16-bit lanes holding whole code bytes: pairs (l', l'+1)
      uint32_t p0 = vperm(0u, qv.x, 0x0C010C00u), p1 = vperm(0u, qv.x, 0x0C030C02u);
      uint32_t p2 = vperm(0u, qv.y, 0x0C010C00u), p3 = vperm(0u, qv.y, 0x0C030C02u);
      uint32_t S = vperm(sv.y, sv.x, ssel);
      float A = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const uint32_t mk = 0x00030003u << (2 * s);
        float t = dot2_f16(p0 & mk, hr[k][4 * s], 0.0f);
        t = dot2_f16(p1 & mk, hr[k][4 * s + 1], t);
        t = dot2_f16(p2 & mk, hr[k][4 * s + 2], t);
        t = dot2_f16(p3 & mk, hr[k][4 * s + 3], t);
        float sc = (float)((S >> (8 * s)) & 0xFu);
        A = fmaf(sc, t, A);
      }
      // mins: high nibbles as binary16 subnormals 16*m, against X_s/16
      uint32_t m01 = vperm(0u, S, 0x0C010C00u) & 0x00F000F0u;
      uint32_t m23 = vperm(0u, S, 0x0C030C02u) & 0x00F000F0u;
      float Bm = dot2_f16(m01, xs[k][0], 0.0f);
      Bm = dot2_f16(m23, xs[k][1], Bm);
      float d = f16_bits_to_f32(dd & 0xFFFFu), dmin = f16_bits_to_f32(dd >> 16);
      float p = fmaf(-dmin, Bm, d * A);
      acc = fmaf(wk[k], p, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      if (residual) residual[row] += acc;
      else out[row] = acc;
    }
  }
}

}  // namespace ds4
