// ffn_b1.hip -- batch-1 decode matvecs for the V4-Flash expert shape
// (hidden 4096, intermediate 2048, IQ2_XXS gate/up, Q2_K down), gfx950.
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, section
// "MoE FFN 部の中身": E(x) = W_down (SiLU(W_gate x) * W_up x), y = sum_k g_k E_k.
// Formats: DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec,
// sections 3 (Q2_K, 84 B / 256) and 4 (IQ2_XXS, 66 B / 256).
//
// At batch 1 every weight byte is used once, so these kernels stream HBM;
// they must keep enough loads in flight to cover the memory latency and keep
// the work per weight value near one VALU op.  Design:
//  * Each wave issues the loads of all its rows before doing anything else;
//    the activation is staged once per workgroup in LDS and each lane keeps
//    its slice in registers (a lane always covers the same columns).
//  * gate/up: an IQ2_XXS grid entry becomes four bf16 pairs from a 4 KB LDS
//    table, a 7-bit sign mask (with its even-parity eighth bit) becomes four
//    XOR masks from a 2 KB LDS table, and v_dot2_f32_bf16 multiplies them with
//    the bf16 activation.  Grid values (< 128) are exact in bf16, so the
//    products are exact and only the fp32 accumulation rounds.  The group
//    scale d*(2s+1)/8 multiplies each 32-value partial sum once.
//  * The SwiGLU output leaves gate/up as 16-bit fixed point with one scale per
//    32 values, grouped exactly as the down matvec's lanes consume it.
//  * down: a Q2_K code is masked in place inside a 16-bit lane (value 4^s q),
//    v_dot2_i32_i16 multiplies it with the fixed-point h exactly, the 4^s is
//    shifted out of the 8-value sum, and the sub-block scale and min are
//    applied with integer multiply-adds; one fp32 conversion per row segment.
//    Each wave handles one routed slot; the six slot partials of a row are
//    added in a fixed order through LDS.
//  * Row reductions use DPP inside rows of 16 lanes and four readlanes.
#include "dev_common.h"

namespace ds4 {

constexpr int kH = 4096;        // hidden size of the fast path
constexpr int kI = 2048;        // intermediate size of the fast path
constexpr int kRowIq2 = 16 * kIq2Bytes;  // 1056 bytes per gate/up row
constexpr int kRowQ2k = 8 * kQ2kBytes;   // 672 bytes per down row

// ---------------------------------------------------------------------------
// SwiGLU output hand-off between the two kernels.  The down matvec gives lane
// L = 8b + 4hh + c of a wave the 32 columns  i = 256b + 128hh + 32s + 8c + j
// (s, j < 4, 8) of every row.  The gate/up kernel therefore computes exactly
// those 32 rows in one workgroup and stores them as 16-bit fixed point with
// one scale per chunk: h_i ~= S * n_i, n_i = round(32767 h_i / max|h|).
// Record per (slot k, lane L), 24 dwords:
//   [0..15]  n as int16 pairs, dword 4s+m = (n[8s+2m], n[8s+2m+1])
//   [16..19] X_s = sum_j n[8s+j]      (int32, for the min term)
//   [20]     S                        (fp32)
// The relative quantisation error (< 2^-16 of the chunk maximum) is eight
// times below that of binary16 rounding, and every later product is exact.
constexpr int kHqDwords = 24;

// LDS tables: grid entry -> 4 bf16 pairs (16 B); 7-bit sign mask -> 4 XOR
// masks (16 B).  The lookups are random, so each table is stored 8 times:
// copy p of entry e sits at 16-byte slot 8e + p, i.e. always in bank group p,
// and lane l reads copy l % 8.  Eight consecutive lanes then touch eight
// different bank groups whatever their indices: the reads are conflict-free.
// Built by 512 threads.
__device__ inline void build_iq2_tables8(const uint8_t* grid, uint4* gt8, uint4* mt8) {
  const int t = threadIdx.x;
  {
    const int e = t >> 1;
    const uint8_t* g = grid + 8 * e;
    uint32_t w[4];
    for (int m = 0; m < 4; m++) {
      uint32_t lo = __float_as_uint((float)g[2 * m]) >> 16;
      uint32_t hi = __float_as_uint((float)g[2 * m + 1]) >> 16;
      w[m] = lo | (hi << 16);
    }
    const uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
    for (int q = 0; q < 4; q++) gt8[8 * e + 4 * (t & 1) + q] = v;
  }
  if (t < 256) {
    const int e = t >> 1;
    uint32_t s8 = (uint32_t)e | ((uint32_t)(__popc(e) & 1) << 7);
    uint32_t w[4];
    for (int m = 0; m < 4; m++)
      w[m] = (((s8 >> (2 * m)) & 1u) << 15) | (((s8 >> (2 * m + 1)) & 1u) << 31);
    const uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
    for (int q = 0; q < 4; q++) mt8[8 * e + 4 * (t & 1) + q] = v;
  }
}

// Raw bytes of one lane's IQ2_XXS row segment: block b = lane/4, groups
// 2j, 2j+1 (j = lane%4), i.e. 64 columns from 256b + 64j.  The 16 group bytes
// start 2 bytes into a 4-byte word for even b; five aligned dwords cover
// them, and the fifth is fetched from inside the group when not needed so the
// last row of a tensor is never overrun.
struct Iq2Seg {
  uint32_t w0, w1, w2, w3, w4, dw;
};

__device__ inline void iq2_load(const uint8_t* row, int lane, Iq2Seg& sg) {
  const int b = lane >> 2, j = lane & 3;
  const uint8_t* blk = row + b * kIq2Bytes;
  const uint8_t* ga = blk + 2 + 16 * j;
  // pointer arithmetic (not integer casts) keeps these global-memory loads
  const uint32_t sh = (uint32_t)((uintptr_t)ga & 3);
  const uint32_t* gp = (const uint32_t*)(ga - sh);
  sg.w0 = gp[0];
  sg.w1 = gp[1];
  sg.w2 = gp[2];
  sg.w3 = gp[3];
  sg.w4 = gp[sh ? 4 : 3];
  sg.dw = *(const uint32_t*)(blk - ((uintptr_t)blk & 3));
}

__device__ inline float iq2_dot(const Iq2Seg& sg, int lane, const uint32_t* xr, const uint4* gt8,
                                const uint4* mt8) {
  const int rep = lane & 7;
  const int b = lane >> 2;
  // block start parity decides both misalignments (rows are 16-byte aligned)
  const uint32_t sh = (b & 1) ? 0u : 2u;
  float d = f16_bits_to_f32(sh ? (sg.dw & 0xFFFFu) : (sg.dw >> 16));
  uint32_t g[4];
  g[0] = align_bytes(sg.w1, sg.w0, sh);
  g[1] = align_bytes(sg.w2, sg.w1, sh);
  g[2] = align_bytes(sg.w3, sg.w2, sh);
  g[3] = align_bytes(sg.w4, sg.w3, sh);
  float acc = 0.0f;
#pragma unroll
  for (int grp = 0; grp < 2; grp++) {
    uint32_t idxw = g[2 * grp], sw = g[2 * grp + 1];
    float dg = d * (float)(2u * (sw >> 28) + 1u) * 0.125f;
    float gacc = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      uint4 gv = gt8[8 * ((idxw >> (8 * kk)) & 0xFFu) + rep];
      uint4 mv = mt8[8 * ((sw >> (7 * kk)) & 0x7Fu) + rep];
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

// Max over the 64 lanes (result in every lane).
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// gate/up + SwiGLU + fixed-point hand-off for one token.
// Grid K*64 workgroups of 512 threads: workgroup (k, L) computes the 32 rows
// of down-lane L for routed slot k; wave w does rows j = 4(w&1)..+3 of
// bit-pair s = w/2.  All weight loads of a wave are issued before anything
// else so that their latency overlaps the table build and the x staging.
__global__ __launch_bounds__(512) void k_gateup_iq2_b1(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ gate,
                                                       const uint8_t* __restrict__ up,
                                                       const uint8_t* __restrict__ grid,
                                                       const int32_t* __restrict__ ids, int E,
                                                       uint32_t* __restrict__ hq,
                                                       uint32_t* status) {
  __shared__ uint4 gt8[256 * 8];
  __shared__ uint4 mt8[128 * 8];
  __shared__ uint4 xs[kH / 8];
  __shared__ float hv[32];
  const int k = blockIdx.x >> 6, L = blockIdx.x & 63;
  const int b = L >> 3, hh = (L >> 2) & 1, c = L & 3;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, s = w >> 1;
  int e = ids[k];
  if (e < 0 || e >= E) {
    if (tid == 0 && L == 0) raise_fault(status, DS4MOE_FAULT_BAD_ID);
    e = 0;
  }
  const int i0 = 256 * b + 128 * hh + 32 * s + 8 * c + 4 * (w & 1);
  Iq2Seg sg[4], su[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    iq2_load(gate + ((size_t)e * kI + i0 + r) * kRowIq2, lane, sg[r]);
    iq2_load(up + ((size_t)e * kI + i0 + r) * kRowIq2, lane, su[r]);
  }
  // x staged in LDS with 16-byte chunk c stored at slot c ^ ((c >> 3) & 7), so
  // the eight chunks a lane reads land in eight bank groups across lanes
  xs[tid ^ ((tid >> 3) & 7)] = ((const uint4*)x)[tid];
  build_iq2_tables8(grid, gt8, mt8);
  __syncthreads();
  uint32_t xr[32];
  {
    const int c0 = 32 * (lane >> 2) + 8 * (lane & 3);
    const int swz = (c0 >> 3) & 7;
#pragma unroll
    for (int q = 0; q < 8; q++) {
      uint4 v = xs[c0 + (q ^ swz)];
      xr[4 * q] = v.x;
      xr[4 * q + 1] = v.y;
      xr[4 * q + 2] = v.z;
      xr[4 * q + 3] = v.w;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float g = wave_sum(iq2_dot(sg[r], lane, xr, gt8, mt8));
    float u = wave_sum(iq2_dot(su[r], lane, xr, gt8, mt8));
    if (lane == 0) hv[8 * s + 4 * (w & 1) + r] = silu(g) * u;
  }
  __syncthreads();
  if (w != 0) return;
  // fixed-point quantisation of the 32 values (lanes 0..31 of wave 0)
  float h = lane < 32 ? hv[lane] : 0.0f;
  float m = wave_max(fabsf(h));
  if (!(m <= 3.0e38f)) raise_fault(status, DS4MOE_FAULT_F16_RANGE);
  float inv = m > 0.0f ? 1.0f / m : 0.0f;
  float hn = h * inv;
  float hp = dpp_f32<0xB1>(hn);  // partner lane t^1
  int pk = __builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(hn, hp));
  int n = (int)(short)(pk & 0xFFFF);
  // X_s: sums of n over aligned groups of 8 lanes
  int xsum = n;
  xsum += __builtin_amdgcn_mov_dpp(xsum, 0xB1, 0xF, 0xF, false);
  xsum += __builtin_amdgcn_mov_dpp(xsum, 0x4E, 0xF, 0xF, false);
  xsum += __builtin_amdgcn_mov_dpp(xsum, 0x141, 0xF, 0xF, false);
  uint32_t* rec = hq + ((size_t)k * 64 + L) * kHqDwords;
  if (lane < 32 && (lane & 1) == 0) rec[lane >> 1] = (uint32_t)pk;
  if (lane < 32 && (lane & 7) == 0) rec[16 + (lane >> 3)] = (uint32_t)xsum;
  if (lane == 0) rec[20] = __float_as_uint(m * (1.0f / 32767.0f));
}

// down + weighted combine (+ residual) for one token.
// Grid H/8 workgroups of 6 waves: wave k handles routed slot k for 8 rows.
__global__ __launch_bounds__(384) void k_down_q2k_b1(const uint32_t* __restrict__ hq,
                                                     const uint8_t* __restrict__ down,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ wts, int E,
                                                     float* __restrict__ out,
                                                     float* __restrict__ residual,
                                                     uint32_t* status) {
  constexpr int R = 8;
  __shared__ float part[6][R];
  const int tid = threadIdx.x, lane = tid & 63, k = tid >> 6;
  const int b = lane >> 3, q8 = lane & 7, hh = q8 >> 2, c = q8 & 3;
  int e = ids[k];
  if (e < 0 || e >= E) {
    if (lane == 0 && blockIdx.x == 0) raise_fault(status, DS4MOE_FAULT_BAD_ID);
    e = 0;
  }
  const int row0 = blockIdx.x * R;
  const uint8_t* base = down + ((size_t)e * kH + row0) * kRowQ2k + b * kQ2kBytes;
  const int qoff = 16 + 32 * hh + 8 * c, soff = 8 * hh;
  uint2 qv[R], sv[R];
  uint32_t dd[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const uint8_t* blk = base + r * kRowQ2k;
    qv[r] = *(const uint2*)(blk + qoff);
    sv[r] = *(const uint2*)(blk + soff);
    dd[r] = *(const uint32_t*)(blk + 80);
  }
  const uint4* rp = (const uint4*)(hq + ((size_t)k * 64 + lane) * kHqDwords);
  uint32_t nr[16];
  int xn[4];
  float S;
  {
    uint4 v0 = rp[0], v1 = rp[1], v2 = rp[2], v3 = rp[3], v4 = rp[4], v5 = rp[5];
    nr[0] = v0.x; nr[1] = v0.y; nr[2] = v0.z; nr[3] = v0.w;
    nr[4] = v1.x; nr[5] = v1.y; nr[6] = v1.z; nr[7] = v1.w;
    nr[8] = v2.x; nr[9] = v2.y; nr[10] = v2.z; nr[11] = v2.w;
    nr[12] = v3.x; nr[13] = v3.y; nr[14] = v3.z; nr[15] = v3.w;
    xn[0] = (int)v4.x; xn[1] = (int)v4.y; xn[2] = (int)v4.z; xn[3] = (int)v4.w;
    S = __uint_as_float(v5.x);
  }
  const float wS = wts[k] * S;
  const uint32_t cb = (uint32_t)(c >> 1);
  const uint32_t ssel = cb | ((cb + 2) << 8) | ((cb + 4) << 16) | ((cb + 6) << 24);
#pragma unroll
  for (int r = 0; r < R; r++) {
    uint32_t p0 = vperm(0u, qv[r].x, 0x0C010C00u), p1 = vperm(0u, qv[r].x, 0x0C030C02u);
    uint32_t p2 = vperm(0u, qv[r].y, 0x0C010C00u), p3 = vperm(0u, qv[r].y, 0x0C030C02u);
    uint32_t S4 = vperm(sv[r].y, sv[r].x, ssel);
    int A = 0, B = 0;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint32_t mk = 0x00030003u << (2 * s);
      int t = sdot2(p0 & mk, nr[4 * s], 0);
      t = sdot2(p1 & mk, nr[4 * s + 1], t);
      t = sdot2(p2 & mk, nr[4 * s + 2], t);
      t = sdot2(p3 & mk, nr[4 * s + 3], t);
      t >>= 2 * s;  // codes were read in place, i.e. times 4^s; exact
      A += (int)((S4 >> (8 * s)) & 0xFu) * t;
      B += (int)((S4 >> (8 * s + 4)) & 0xFu) * xn[s];
    }
    float d = f16_bits_to_f32(dd[r] & 0xFFFFu), dmin = f16_bits_to_f32(dd[r] >> 16);
    float p = wS * fmaf(-dmin, (float)B, d * (float)A);
    p = wave_sum(p);
    if (lane == 0) part[k][r] = p;
  }
  __syncthreads();
  if (tid < R) {
    float acc = ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) +
                (part[4][tid] + part[5][tid]);
    if (residual) residual[row0 + tid] += acc;
    else out[row0 + tid] = acc;
  }
}

}  // namespace ds4
