// ffn_q4k.hip -- batch-1 decode matvecs for Q4_K expert matrices with the
// V4-Flash expert shape (hidden 4096, intermediate 2048), gfx950.  They pair
// with the IQ2_XXS / Q2_K kernels of ffn_b1.hip: a layer's gate/up and down
// kernels are chosen by format, and both sides exchange the fp32 SwiGLU
// rows [token][6][2048].
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, section
// "MoE FFN 部の中身".  Format: DS4C2 = qiita.com/yoshiyakato/items/
// 4678be0e7860ddb444ec, section 3 (type table: Q4_K, 144 B / 256 values;
// affine per sub-block, FLOW quantisation section); layout of the k-quant
// family: fp16 d, fp16 dmin, 12 bytes of 6-bit scale/min per 32-value
// sub-block, 128 bytes of 4-bit codes (byte 16 + 32c + l: value 64c + l in
// the low nibble, 64c + 32 + l in the high nibble).
//
// A lane always covers the same 64 consecutive values of a row: chunk c of
// block b (lane L: b = L >> 2 of the 16 blocks of a 4096-value row, c = L & 3),
// i.e. the 32 code bytes at 16 + 32c and dword c of the block's 16-byte
// header; the four lanes of a block exchange their header dwords with DPP
// quad permutes when the row is used, so a row costs a lane 9 registers.  The lane's activations are held as 16-bit fixed
// point with one scale (x ~= S n, n = round(32767 x / max|x|), error below
// 2^-16 of the lane's maximum), paired as the code bytes pair up inside
// 16-bit lanes: a code dword w holds bytes (4k .. 4k+3), so w & 0x000F000F
// are the low-nibble codes of values 4k and 4k+2, (w >> 8) & 0x000F000F those
// of 4k+1 and 4k+3, and the 0x00F000F0 masks give 16 times the high-nibble
// codes.  v_dot2_i32_i16 multiplies them exactly; the sub-block scales and
// mins are applied once per row segment in fp32.
#include "dev_common.h"

namespace ds4 {

constexpr int kRowQ4kGu = 16 * kQ4kBytes;  // 2304 bytes per gate/up row
constexpr int kRowQ4kDn = 8 * kQ4kBytes;   // 1152 bytes per down row

struct Q4Seg {
  uint32_t hw;   // dword c of the header (d | dmin << 16, then the 12 scale/min bytes)
  uint4 c0, c1;  // the 32 code bytes of the lane's chunk
};

__device__ inline void q4k_load(const uint8_t* __restrict__ row, int b, int c, Q4Seg& s) {
  const uint8_t* blk = row + kQ4kBytes * b;  // 144 = 9 * 16: 16-byte aligned
  s.hw = *(const uint32_t*)(blk + 4 * c);
  s.c0 = *(const uint4*)(blk + 16 + 32 * c);
  s.c1 = *(const uint4*)(blk + 32 + 32 * c);
}

// dword J of the header, from lane J of the lane's quad (all four lanes of a
// quad are active wherever a row is used)
template <int J>
__device__ inline uint32_t q4k_hdr(uint32_t hw) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)hw, J * 0x55, 0xF, 0xF, false);  // quad_perm [J,J,J,J]
}

// A lane's 64 activations as fixed point: xl[2k], xl[2k+1] pair values
// (4k, 4k+2) and (4k+1, 4k+3) of the low half, xh likewise for values
// 32 + ..; sl, sh = sums of the low and high halves; returns the scale S.
// val(i) gives value i (read twice: for the maximum, then for the packing,
// so that the 64 values need not be held at once).
// A NaN or infinite value makes S NaN, so that every product of the lane is
// NaN, as the exact products would be (the fixed point cannot carry it).
template <class V>
__device__ inline float q4k_fix(V val, uint32_t* xl, uint32_t* xh, int& sl, int& sh) {
  AbsMax am;
#pragma unroll
  for (int i = 0; i < 64; i++) am.add(val(i));
  bool nonfinite;
  const float mx = am.value(nonfinite);
  const float inv = mx > 0.0f ? 1.0f / mx : 0.0f;
  auto pk = [&](int i, int j) {
    return (uint32_t)__builtin_bit_cast(int, __builtin_amdgcn_cvt_pknorm_i16(val(i) * inv, val(j) * inv));
  };
#pragma unroll
  for (int k = 0; k < 8; k++) {
    xl[2 * k] = pk(4 * k, 4 * k + 2);
    xl[2 * k + 1] = pk(4 * k + 1, 4 * k + 3);
    xh[2 * k] = pk(32 + 4 * k, 32 + 4 * k + 2);
    xh[2 * k + 1] = pk(32 + 4 * k + 1, 32 + 4 * k + 3);
  }
  int a = 0, b = 0;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    a = sdot2(xl[q], 0x00010001u, a);
    b = sdot2(xh[q], 0x00010001u, b);
  }
  sl = a;
  sh = b;
  return nonfinite ? __builtin_nanf("") : mx * (1.0f / 32767.0f);
}

// Partial dot product of a lane's 64 values of one row with the fixed-point
// activations (before the lane's scale S).  c: the lane's chunk.
__device__ inline float q4k_dot64(const Q4Seg& s, int c, const uint32_t* xl, const uint32_t* xh,
                                  int sl, int sh) {
  const uint32_t w[8] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w, s.c1.x, s.c1.y, s.c1.z, s.c1.w};
  int al = 0, ah = 0;  // |al| < 2^24; ah = 16 x the high-half sum, |ah| < 2^28
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const uint32_t w8 = w[k] >> 8;
    al = sdot2(w[k] & 0x000F000Fu, xl[2 * k], al);
    al = sdot2(w8 & 0x000F000Fu, xl[2 * k + 1], al);
    ah = sdot2(w[k] & 0x00F000F0u, xh[2 * k], ah);
    ah = sdot2(w8 & 0x00F000F0u, xh[2 * k + 1], ah);
  }
  // scale and min of sub-blocks j0 = 2c, j1 = 2c + 1 (6-bit fields)
  const uint32_t hx = q4k_hdr<0>(s.hw), hy = q4k_hdr<1>(s.hw), hz = q4k_hdr<2>(s.hw),
                 hv = q4k_hdr<3>(s.hw);
  const uint32_t t = 16u * (uint32_t)(c & 1);  // byte 2(c & 1) of the dwords, as a bit offset
  const uint32_t y2 = hy >> t, z2 = hz >> t, w2 = hv >> t;
  // chunks 0, 1: six bits of bytes 4..11; chunks 2, 3: a nibble of bytes
  // 12..15 and the top two bits of bytes 4..11 (as bits 4, 5).  Written
  // without a branch on the lane's chunk, so that nothing per row is hoisted.
  const bool hi = c >= 2;
  const uint32_t mlo = hi ? 15u : 63u, mhi = hi ? 0x30u : 0u;
  const uint32_t srs = hi ? w2 : y2, srm = hi ? (w2 >> 4) : z2;
  const int sc0 = (int)((srs & mlo) | ((y2 >> 2) & mhi));
  const int sc1 = (int)(((srs >> 8) & mlo) | ((y2 >> 10) & mhi));
  const int m0 = (int)((srm & mlo) | ((z2 >> 2) & mhi));
  const int m1 = (int)(((srm >> 8) & mlo) | ((z2 >> 10) & mhi));
  const float d = f16_bits_to_f32(hx & 0xFFFFu), dmin = f16_bits_to_f32(hx >> 16);
  const float main = (float)sc0 * (float)al + (float)sc1 * (float)(ah >> 4);  // ah is a multiple of 16
  const int mins = __mul24(m0, sl) + __mul24(m1, sh);  // |sl|, |sh| < 2^21
  return fmaf(d, main, -dmin * (float)mins);
}

// gate/up + SwiGLU for one token, Q4_K gate and up.  Grid (256, T) of 16
// waves; wave w of workgroup g handles flattened rows 3u .. 3u+2, u = 16g + w,
// of the six routed slots (as k_gateup_b1); with SEL the workgroup first picks
// the top-6 experts from the router's key intervals (wave 0).  Each lane reads
// its own 64 activations (from L2: 128 bytes) and turns them into fixed point
// before any weight is requested, so that only the fixed-point form is live
// beside the three rows' weights.  Writes the fp32 SwiGLU rows
// [token][6][2048].
template <bool SEL>
__global__ __launch_bounds__(kGuWaves * 64) void k_gateup_q4k_b1(GateUpB1Args a) {
  __shared__ int sel_e[8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = (blockIdx.x * kGuWaves + w) * kGuRows;  // flattened
  const int tok = blockIdx.y;
  const uint16_t* xtok = a.x + (size_t)tok * kH;
  const int32_t* idtok = a.ids + 6 * tok;
  float* htok = a.h + (size_t)tok * 6 * kI;
  const int b = lane >> 2, c = lane & 3;

  // the lane's 64 values 256b + 64c .. +63 (bf16), then fixed point
  uint32_t xl[16], xh[16];
  int sl, sh;
  float S;
  SelIds sel{0, 0.0f, false};
  const float4* kbt = a.kbuf + (size_t)blockIdx.y * a.E;
  {
    const uint4* xp = (const uint4*)(xtok + 256 * b + 64 * c);
    uint4 xq[8];
#pragma unroll
    for (int q = 0; q < 8; q++) xq[q] = xp[q];
    if (SEL && w == 0) {
      const RouteSrc src{xtok, DS4MOE_BF16, a.rw, a.rw_dt, a.rbias, kH};
      sel = select_ids(kbt, a.E, 6, a.status, blockIdx.x == 0, src);
      if (lane < 6) sel_e[lane] = sel.e;
    }
    auto xval = [&](int i) {  // value i of the lane's 64 (bf16 pairs in xq)
      const uint4 q = xq[i >> 3];
      const uint32_t ww = (i & 6) == 0 ? q.x : (i & 6) == 2 ? q.y : (i & 6) == 4 ? q.z : q.w;
      return bf16_bits_to_f32((i & 1) ? (ww >> 16) : (ww & 0xFFFFu));
    };
    S = q4k_fix(xval, xl, xh, sl, sh);
    // materialise the fixed-point form here, before the weight loads, so
    // that the raw values are dead by then (bounded registers)
#pragma unroll
    for (int q = 0; q < 16; q++) asm volatile("" ::"v"(xl[q]), "v"(xh[q]));
  }
  __builtin_amdgcn_sched_barrier(0);
  if (SEL) __syncthreads();  // sel_e visible

  Q4Seg sg[kGuRows], su[kGuRows];
#pragma unroll
  for (int r = 0; r < kGuRows; r++) {
    const int k = (row0 + r) >> 11;
    int e = SEL ? __builtin_amdgcn_readfirstlane(sel_e[k]) : load_scalar_i32(idtok, k);
    if (e < 0 || e >= a.E) {
      if (lane == 0 && ((row0 + r) & (kI - 1)) == 0) raise_fault(a.status, DS4MOE_FAULT_BAD_ID);
      e = 0;
    }
    const size_t rowi = (size_t)e * kI + ((row0 + r) & (kI - 1));
    q4k_load(a.gate + rowi * kRowQ4kGu, b, c, sg[r]);
    q4k_load(a.up + rowi * kRowQ4kGu, b, c, su[r]);
  }
  // the gates, off the path to the first weight request; workgroup 0 of each
  // row publishes the token's ids and gates
  if (SEL && w == 0 && blockIdx.x == 0) {
    const float g = select_gate(kbt, 6, a.scale, sel);
    if (lane < 6) {
      a.ids_out[6 * blockIdx.y + lane] = sel.e;
      a.wts_out[6 * blockIdx.y + lane] = g;
    }
  }
  float v[8];
#pragma unroll
  for (int r = 0; r < kGuRows; r++) {  // one row at a time: bounded registers
    v[r] = S * q4k_dot64(sg[r], c, xl, xh, sl, sh);
    __builtin_amdgcn_sched_barrier(0);
    v[4 + r] = S * q4k_dot64(su[r], c, xl, xh, sl, sh);
    __builtin_amdgcn_sched_barrier(0);
  }
  v[3] = 0.0f;
  v[7] = 0.0f;
  const float tot = reduce8(v);
  // lane 16*rho holds the gate total of row c[rho]; its up total sits 8 lanes
  // further on (c = {0,2,1,3}; row 3 is padding)
  const float upv = dpp_f32<0x128>(tot);
  if ((lane & 15) == 0 && lane != 48) {
    const int rho = lane >> 4;
    const int r = (rho == 1) ? 2 : (rho == 2) ? 1 : rho;
    htok[row0 + r] = silu(tot) * upv;
  }
}

// down + weighted combine (+ residual) for one token, Q4_K down.  Grid
// (H / 16, T), 12 waves (as k_down_q2k_b1): wave w handles routed slot
// k = w / 2 for eight rows, two rows per step (lanes 0-31 the even row,
// 32-63 the odd one); lane 32u + L covers the 64 values of chunk L & 3 of
// block L >> 2 of its row.  The token's six SwiGLU rows are staged in LDS
// before any weight is requested.
__global__ __launch_bounds__(kDnThreads) void k_down_q4k_b1(const float* __restrict__ h,
                                                            const uint8_t* __restrict__ down,
                                                            const int32_t* __restrict__ ids,
                                                            const float* __restrict__ wts, int E,
                                                            float* __restrict__ out,
                                                            float* __restrict__ residual,
                                                            uint32_t* status) {
  constexpr int R = kDnRows;
  constexpr int kChunks = 6 * kI / 4;  // 16-byte chunks of h
  __shared__ float4 hs[kChunks];       // 48 KB
  __shared__ float part[6][kDnBlockRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = w >> 1, rh = w & 1;
  const int u = lane >> 5, L = lane & 31, b = L >> 2, c = L & 3;
  const int tok = blockIdx.y;
  h += (size_t)tok * 6 * kI;
  ids += 6 * tok;
  wts += 6 * tok;
  if (out) out += (size_t)tok * kH;
  if (residual) residual += (size_t)tok * kH;
  int e = load_scalar_i32(ids, k);
  const float wk = __int_as_float(load_scalar_i32((const int32_t*)wts, k));
  // the residual rows this workgroup adds to, requested before anything else:
  // read at the end, their round trip came after all the arithmetic
  float res_in = 0.0f;
  if (residual && tid < kDnBlockRows) res_in = residual[blockIdx.x * kDnBlockRows + tid];
  static_assert(kChunks == 4 * kDnThreads, "four h chunks per thread");
  const float4* hg = (const float4*)h + tid;
  const float4 hc0 = hg[0], hc1 = hg[kDnThreads], hc2 = hg[2 * kDnThreads], hc3 = hg[3 * kDnThreads];
  auto put = [&](int q, float4 v) {
    const int G = tid + kDnThreads * q;
    hs[(G & ~511) | dn_chunk(G & 511)] = v;
  };
  put(0, hc0);
  put(1, hc1);
  put(2, hc2);
  put(3, hc3);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const bool bad_id = e < 0 || e >= E;
  e = bad_id ? 0 : e;
  const int row0 = blockIdx.x * kDnBlockRows + rh * R;
  const uint8_t* base = down + ((size_t)e * kH + row0 + u) * kRowQ4kDn;
  Q4Seg sg[R / 2];
#pragma unroll
  for (int m = 0; m < R / 2; m++) q4k_load(base + 2 * m * kRowQ4kDn, b, c, sg[m]);
  // this lane's 64 values of slot k: h[k][256b + 64c .. +63]
  uint32_t xl[16], xh[16];
  int sl, sh;
  float S;
  {
    float hv[64];
    const int G0 = 64 * b + 16 * c;  // chunk of value 256b + 64c
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const float4 f = hs[512 * k + dn_chunk(G0 + q)];
      hv[4 * q] = f.x;
      hv[4 * q + 1] = f.y;
      hv[4 * q + 2] = f.z;
      hv[4 * q + 3] = f.w;
    }
    S = q4k_fix([&](int i) { return hv[i]; }, xl, xh, sl, sh);
  }
  const float wS = wk * S;
  float pr[R / 2];
#pragma unroll
  for (int m = 0; m < R / 2; m++) pr[m] = wS * q4k_dot64(sg[m], c, xl, xh, sl, sh);
  const float tot = reduce4x2(pr);
  if ((lane & 7) == 0) {
    const int rho = lane >> 4, up8 = (lane >> 3) & 1;
    const int m = (rho & 1) + 2 * up8, uu = rho >> 1;
    part[k][rh * R + 2 * m + uu] = tot;
  }
  __syncthreads();
  if (tid < kDnBlockRows) {
    float acc = ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) +
                (part[4][tid] + part[5][tid]);
    const int row = blockIdx.x * kDnBlockRows + tid;
    if (residual) residual[row] = res_in + acc;
    else out[row] = acc;
  }
  if (bad_id && lane == 0 && blockIdx.x == 0 && rh == 0) raise_fault(status, DS4MOE_FAULT_BAD_ID);
}

}  // namespace ds4
