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
//  * The SwiGLU output leaves gate/up in fp32; each down lane turns the 64
//    values it consumes into 16-bit fixed point with one scale (their
//    largest magnitude).
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
// gate/up LDS tables, one copy per workgroup:
//   signs: 7-bit sign field s (with its even-parity eighth bit) as four XOR
//          masks on bf16 pairs, stored 16 times, copy p at (s << 8) | (p << 4);
//   grid:  entry e (8 grid values as four bf16 pairs, 16 B) stored 16 times,
//          copy p at 32 KB + (e << 8) | (p << 4).
// Lane l reads copy l % 16.  A 16-byte LDS read serves 16 lanes per clock
// from 16 distinct 16-byte bank groups, so these random lookups never
// conflict, and both addresses are formed by one or two VALU ops (the grid
// index byte is moved to bits 8..15 by v_perm); the table bases sit in the
// 16-bit offset field of the LDS reads.
constexpr int kSignTab = 128 * 256;                // 32 KB
constexpr int kGridTab = 256 * 256;                // 64 KB

__device__ inline uint4 grid_pairs(uint2 g) {
  uint32_t w[4];
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const uint32_t word = m < 2 ? g.x : g.y;
    const float lo = (float)((word >> (16 * (m & 1))) & 0xFFu);
    const float hi = (float)((word >> (16 * (m & 1) + 8)) & 0xFFu);
    w[m] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ inline uint4 sign_masks(int s7) {
  const uint32_t s8 = (uint32_t)s7 | ((uint32_t)(__popc(s7) & 1) << 7);
  uint32_t w[4];
#pragma unroll
  for (int m = 0; m < 4; m++)
    w[m] = (((s8 >> (2 * m)) & 1u) << 15) | (((s8 >> (2 * m + 1)) & 1u) << 31);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Raw bytes of one lane's IQ2_XXS row segment: block b = lane/4, groups
// 2j, 2j+1 (j = lane%4), i.e. 64 columns from 256b + 64j.  The 16 group bytes
// start 2 bytes into a 4-byte word for even b; five aligned dwords cover
// them, and the fifth is fetched from inside the group when not needed so the
// last row of a tensor is never overrun.  dw is the aligned word holding the
// block scale d.  Offsets are in dwords from the (wave-uniform) row start.
struct Iq2Seg {
  uint32_t w0, w1, w2, w3, w4, dw;
};
struct Iq2Off {
  uint32_t o0, o4, od;
};

__device__ inline Iq2Off iq2_offsets(int lane) {
  const int b = lane >> 2, j = lane & 3;
  const uint32_t start = (uint32_t)(kIq2Bytes * b + 2 + 16 * j);
  Iq2Off o;
  o.o0 = start >> 2;
  o.o4 = o.o0 + ((start & 3) ? 4u : 3u);
  o.od = (uint32_t)(kIq2Bytes * b) >> 2;
  return o;
}

// Row r of a wave's rows (rows are kRowIq2 = 264 dwords apart).
__device__ inline void iq2_load(const uint32_t* __restrict__ base, int r, const Iq2Off& o,
                                Iq2Seg& sg) {
  const uint32_t* p = base + r * (kRowIq2 / 4);
  sg.w0 = p[o.o0];
  sg.w1 = p[o.o0 + 1];
  sg.w2 = p[o.o0 + 2];
  sg.w3 = p[o.o0 + 3];
  sg.w4 = p[o.o4];
  sg.dw = p[o.od];
}

// Partial dot product of one lane's 64 columns with x (bf16 pairs in xr).
// The group scale d(2s+1)/8 is applied as (16s+8) per group and d/64 once.
__device__ inline float iq2_dot16(const Iq2Seg& sg, uint32_t sh, const uint32_t* xr,
                                  const uint8_t* gtab, const uint8_t* stab, uint32_t rep16) {
  const float d = f16_bits_to_f32(sh ? (sg.dw & 0xFFFFu) : (sg.dw >> 16));
  uint32_t g[4];
  g[0] = align_bytes(sg.w1, sg.w0, sh);
  g[1] = align_bytes(sg.w2, sg.w1, sh);
  g[2] = align_bytes(sg.w3, sg.w2, sh);
  g[3] = align_bytes(sg.w4, sg.w3, sh);
  float acc = 0.0f;
#pragma unroll
  for (int grp = 0; grp < 2; grp++) {
    const uint32_t idxw = g[2 * grp], sw = g[2 * grp + 1];
    // all eight table reads of the group first, so that one LDS round trip
    // covers four entries
    uint4 gv[4], mv[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const uint32_t ga = vperm(idxw, rep16, 0x0C0C0000u | ((4u + kk) << 8));
      const uint32_t sa = (((sw >> (7 * kk)) & 0x7Fu) << 8) | rep16;
      gv[kk] = *(const uint4*)(gtab + ga);
      mv[kk] = *(const uint4*)(stab + sa);
    }
    float ga0 = 0.0f, ga1 = 0.0f;  // two chains of dependent dot products
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const uint32_t* xp = xr + grp * 16 + kk * 4;
      float& ac = (kk & 1) ? ga1 : ga0;
      ac = dot2_bf16(gv[kk].x ^ mv[kk].x, xp[0], ac);
      ac = dot2_bf16(gv[kk].y ^ mv[kk].y, xp[1], ac);
      ac = dot2_bf16(gv[kk].z ^ mv[kk].z, xp[2], ac);
      ac = dot2_bf16(gv[kk].w ^ mv[kk].w, xp[3], ac);
    }
    // 16s + 8 from the top nibble: exact in fp32
    acc = fmaf((float)(((sw & 0xF0000000u) | 0x08000000u) >> 24), ga0 + ga1, acc);
  }
  return acc * (d * 0.015625f);
}

// Sums over the 64 lanes of eight per-lane values at once.  Lane L ends up
// holding the total of v[4*((L>>3)&1) + c[L>>4]], c = {0,2,1,3}; every lane
// of an aligned group of 8 holds the same total.  18 VALU ops instead of 8
// separate wave reductions.
__device__ inline float reduce8(const float* v) {
  float u[4];
#pragma unroll
  for (int p = 0; p < 4; p++) {
    // halves: lanes 0-31 <- v[2p] (both halves summed), lanes 32-63 <- v[2p+1]
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * p]),
                                              __float_as_uint(v[2 * p + 1]), false, false);
    u[p] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float w2[2];
#pragma unroll
  for (int q = 0; q < 2; q++) {
    // rows of 16: row 0 <- v[4q], row 1 <- v[4q+2], row 2 <- v[4q+1], row 3 <- v[4q+3]
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[2 * q]),
                                              __float_as_uint(u[2 * q + 1]), false, false);
    w2[q] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // within rows of 16: lanes 0-7 <- w2[0], lanes 8-15 <- w2[1]
  const bool up8 = (threadIdx.x & 8) != 0;
  const float t = up8 ? w2[0] : w2[1];
  float z = (up8 ? w2[1] : w2[0]) + dpp_f32<0x128>(t);  // row_ror:8
  z += dpp_f32<0xB1>(z);
  z += dpp_f32<0x4E>(z);
  z += dpp_f32<0x141>(z);
  return z;
}

struct GateUpB1Args {
  const uint16_t* x;       // [4096] bf16
  const uint8_t* gate;     // [E][2048][1056 B]
  const uint8_t* up;
  const uint8_t* grid;     // [256][8]
  const int32_t* ids;      // [6] (no selection)
  const float4* kbuf;      // [E] key intervals (selection)
  float scale;
  int32_t* ids_out;        // [6] (selection)
  float* wts_out;          // [6] (selection)
  const void* rw;          // router weights [E][4096] and their dtype, and the
  int rw_dt;               // selection bias [E] (selection: for the exact
  const float* rbias;      // recomputation of keys the intervals leave open)
  int E;
  float* h;                // [6][2048] SwiGLU output
  uint32_t* status;
};

constexpr int kDnRows = 8;                                   // down rows per wave
constexpr int kGuWaves = 16;                                  // waves per workgroup
constexpr int kGuRows = 3;                                    // rows (gate + up) per wave
constexpr int kGuBlocks = 6 * kI / (kGuWaves * kGuRows);      // 256
static_assert(kGuBlocks * kGuWaves * kGuRows == 6 * kI, "gate/up rows must tile the 6 slots");
static_assert(384 + kH / 8 <= kGuWaves * 64 - 64, "x staging needs one helper per 16-byte chunk");


// Table build, conflict-free: a thread owns one entry and writes its 16
// copies in the order p = (j + entry) % 16, so the 16 lanes a store serves in
// one clock hit 16 different bank groups.
__device__ inline void store_copies(uint8_t* tab, int entry, uint4 v) {
#pragma unroll
  for (int j = 0; j < 16; j++)
    *(uint4*)(tab + (entry << 8) + (((j + entry) & 15) << 4)) = v;
}

// gate/up + SwiGLU, one grid row of 256 workgroups of 16 waves per token
// (blockIdx.y); wave w of workgroup g handles flattened rows 3u .. 3u+2,
// u = 16g + w, of the six routed slots (row r of slot k is flattened row
// 2048k + r), gate and up.  With SEL the workgroup first picks the token's
// top-6 experts from the router's key intervals (wave 0, while the other
// waves build the tables and stage x); workgroup 0 of each row publishes the
// token's ids and gates for the down kernel.  Without SEL the weight loads
// are issued before the tables are built.
template <bool SEL>
__global__ __launch_bounds__(kGuWaves * 64) void k_gateup_b1(GateUpB1Args a) {
  // one static array so that the table offsets are compile-time constants
  __shared__ uint4 lds4[(kSignTab + kGridTab + 2 * kH) / 16 + 2];
  uint8_t* stab = (uint8_t*)lds4;                        // 32 KB
  uint8_t* gtab = stab + kSignTab;                       // 64 KB
  uint4* xs = lds4 + (kSignTab + kGridTab) / 16;         // 8 KB
  int* sel_e = (int*)(lds4 + (kSignTab + kGridTab + 2 * kH) / 16);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in scalar registers
  const int row0 = (blockIdx.x * kGuWaves + w) * kGuRows;  // flattened
  // token t = blockIdx.y (one grid row per token)
  const int tok = blockIdx.y;
  const uint16_t* xtok = a.x + (size_t)tok * kH;
  const int32_t* idtok = a.ids + 6 * tok;
  float* htok = a.h + (size_t)tok * 6 * kI;
  const Iq2Off off = iq2_offsets(lane);
  Iq2Seg sg[kGuRows], su[kGuRows];

  // helper roles for the table build and x staging; their global loads are
  // issued before the weight loads so that waiting for them never waits for
  // weights (the vector memory counter retires in order)
  const int t = tid - 64;
  uint2 gb = make_uint2(0, 0);
  uint4 xv = make_uint4(0, 0, 0, 0);
  if (t >= 0 && t < 256) gb = *(const uint2*)(a.grid + 8 * t);
  else if (t >= 384 && t < 384 + kH / 8) xv = ((const uint4*)xtok)[t - 384];

  // Expert of each of the wave's rows (wave-uniform), validated.
  auto expert_rows = [&](const int* e_of_slot_lds, uint32_t* erow) {
#pragma unroll
    for (int r = 0; r < kGuRows; r++) {
      const int k = (row0 + r) >> 11;
      int e = SEL ? __builtin_amdgcn_readfirstlane(e_of_slot_lds[k]) : load_scalar_i32(idtok, k);
      if (e < 0 || e >= a.E) {
        if (lane == 0 && ((row0 + r) & (kI - 1)) == 0) raise_fault(a.status, DS4MOE_FAULT_BAD_ID);
        e = 0;
      }
      erow[r] = (uint32_t)e;
    }
  };
  uint32_t erow[kGuRows];
  auto load_row = [&](int r) {
    const size_t rowi = (size_t)erow[r] * kI + ((row0 + r) & (kI - 1));
    iq2_load((const uint32_t*)(a.gate + rowi * kRowIq2), 0, off, sg[r]);
    iq2_load((const uint32_t*)(a.up + rowi * kRowIq2), 0, off, su[r]);
  };
  // Without selection: two rows in flight from the start, the third issued
  // after the table build.
  static_assert(kGuRows == 3, "the load schedule assumes three rows per wave");
  if (!SEL) {
    expert_rows(nullptr, erow);
    load_row(0);
    load_row(1);
  }

  SelIds sel{0, 0.0f, false};
  const float4* kbt = a.kbuf + (size_t)blockIdx.y * a.E;
  if (SEL && w == 0) {
    const RouteSrc src{xtok, DS4MOE_BF16, a.rw, a.rw_dt, a.rbias, kH};
    sel = select_ids(kbt, a.E, 6, a.status, blockIdx.x == 0, src);
    if (lane < 6) sel_e[lane] = sel.e;
  } else if (t >= 0 && t < 256) {
    store_copies(gtab, t, grid_pairs(gb));
  } else if (t >= 256 && t < 384) {
    store_copies(stab, t - 256, sign_masks(t - 256));
  } else if (t >= 384 && t < 384 + kH / 8) {
    // x chunk c (16 B) at slot c ^ ((c >> 3) & 7): a lane's eight chunks
    // then fall in eight bank groups
    const int c = t - 384;
    xs[c ^ ((c >> 3) & 7)] = xv;
  }
  __syncthreads();
  if (SEL) {  // the loads start only now: request all three rows at once
    expert_rows(sel_e, erow);
    load_row(0);
    load_row(1);
    load_row(2);
    // the gates, off the path to the first weight request; workgroup 0 of
    // each row publishes the token's ids and gates
    if (w == 0 && blockIdx.x == 0) {
      const float g = select_gate(kbt, 6, a.scale, sel);
      if (lane < 6) {
        a.ids_out[6 * blockIdx.y + lane] = sel.e;
        a.wts_out[6 * blockIdx.y + lane] = g;
      }
    }
  } else {
    load_row(2);
  }

  uint32_t xr[32];
  {
    const int c0 = 32 * (lane >> 2) + 8 * (lane & 3);
    const int swz = lane & 7;  // (c0 >> 3) & 7
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const uint4 v = xs[c0 + (q ^ swz)];
      xr[4 * q] = v.x;
      xr[4 * q + 1] = v.y;
      xr[4 * q + 2] = v.z;
      xr[4 * q + 3] = v.w;
    }
  }
  // block start parity decides both misalignments (rows are 16-byte aligned)
  const uint32_t sh = ((lane >> 2) & 1) ? 0u : 2u;
  const uint32_t rep16 = (uint32_t)(lane & 15) << 4;
  float v[8];
  v[0] = iq2_dot16(sg[0], sh, xr, gtab, stab, rep16);
  v[4] = iq2_dot16(su[0], sh, xr, gtab, stab, rep16);
#pragma unroll
  for (int r = 1; r < kGuRows; r++) {
    v[r] = iq2_dot16(sg[r], sh, xr, gtab, stab, rep16);
    v[4 + r] = iq2_dot16(su[r], sh, xr, gtab, stab, rep16);
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

// gate/up + SwiGLU for a few tokens, each distinct routed expert read once.
// Grid (kI / kFewFeat, items): work item u is one expert e and the nrows
// (at most 16) sorted pairs that chose it, rows row0 .. row0 + nrows - 1 of
// the permutation (pair p = perm[row] = 6t + k).  Wave w of workgroup b
// takes features f0 = kFewFeat b + 2w and f0 + 1 of expert e, gate and up:
// it requests those four rows before anything else (lane layout of the
// batch-1 kernel: 64 columns per lane), then decodes each 8-value group once
// and multiplies it with the x of every token of the item, kFewTok tokens
// per pass.  The pass's x sits in LDS, 16-byte chunk c of a token at
// c + (c >> 4) (one spare chunk per 16): lane l reads chunks 8l + i (i < 8),
// at 8l + (l >> 1) + i, so the 16 lanes one read serves hit 16 distinct bank
// groups and every address is the lane's base plus an immediate.  The pairs are
// read through the scalar cache, so no wait for them queues behind weights.
// Output: h[p][f] = SiLU(gate) * up in fp32, the batch-1 layout [T][6][kI].
constexpr int kFewWaves = 16;
constexpr int kFewFeat = 2 * kFewWaves;  // features per workgroup
constexpr int kFewTok = 4;               // tokens per pass
constexpr int kXsTok = kH / 8;           // 16-byte chunks of one token's x
constexpr int kXsStride = kXsTok + kXsTok / 16;  // and their LDS slots

struct GateUpFewArgs {
  const uint16_t* x;       // [T][4096] bf16
  const uint8_t* gate;     // [E][2048][1056 B]
  const uint8_t* up;
  const uint8_t* grid;     // [256][8]
  const int32_t* items;    // [n][3]: expert, first sorted row, rows (one item per expert)
  const int32_t* n_items;  // n_items[0]: the number of items
  const int32_t* perm;     // sorted row -> pair 6t + k
  float* h;                // [T*6][2048] by pair
};

// iq2_dot16 for the x of tokens 0 .. nt-1 (xl: the lane's first slot in
// the pass's x, kXsStride slots per token): acc[j] = the lane's partial dot
// product of its 64 columns of the row with token j's x.
template <int NT>
__device__ __attribute__((always_inline)) inline void iq2_dot16_multi(const Iq2Seg& sg, uint32_t sh, const uint4* xl,
                                       const uint8_t* gtab, const uint8_t* stab, uint32_t rep16,
                                       int nt, float (&acc)[NT]) {
  const float d = f16_bits_to_f32(sh ? (sg.dw & 0xFFFFu) : (sg.dw >> 16));
  uint32_t g[4];
  g[0] = align_bytes(sg.w1, sg.w0, sh);
  g[1] = align_bytes(sg.w2, sg.w1, sh);
  g[2] = align_bytes(sg.w3, sg.w2, sh);
  g[3] = align_bytes(sg.w4, sg.w3, sh);
  float a2[NT];
#pragma unroll
  for (int j = 0; j < NT; j++) a2[j] = 0.0f;
#pragma unroll
  for (int grp = 0; grp < 2; grp++) {
    const uint32_t idxw = g[2 * grp], sw = g[2 * grp + 1];
    uint4 gv[4], mv[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const uint32_t ga = vperm(idxw, rep16, 0x0C0C0000u | ((4u + kk) << 8));
      const uint32_t sa = (((sw >> (7 * kk)) & 0x7Fu) << 8) | rep16;
      gv[kk] = *(const uint4*)(gtab + ga);
      mv[kk] = *(const uint4*)(stab + sa);
    }
    // the group's 32 values as bf16 pairs, decoded once for every token
    uint32_t wv[16];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      wv[4 * kk] = gv[kk].x ^ mv[kk].x;
      wv[4 * kk + 1] = gv[kk].y ^ mv[kk].y;
      wv[4 * kk + 2] = gv[kk].z ^ mv[kk].z;
      wv[4 * kk + 3] = gv[kk].w ^ mv[kk].w;
    }
    const float sc = (float)(((sw & 0xF0000000u) | 0x08000000u) >> 24);  // 16s + 8
#pragma unroll
    for (int j = 0; j < NT; j++) {
      if (j < nt) {  // wave-uniform
        float ga0 = 0.0f, ga1 = 0.0f;  // two chains
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
          const uint4 xv = xl[j * kXsStride + 4 * grp + kk];
          float& ac = (kk & 1) ? ga1 : ga0;
          ac = dot2_bf16(wv[4 * kk], xv.x, ac);
          ac = dot2_bf16(wv[4 * kk + 1], xv.y, ac);
          ac = dot2_bf16(wv[4 * kk + 2], xv.z, ac);
          ac = dot2_bf16(wv[4 * kk + 3], xv.w, ac);
        }
        a2[j] = fmaf(sc, ga0 + ga1, a2[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NT; j++) acc[j] = a2[j] * (d * 0.015625f);
}

__global__ __launch_bounds__(kFewWaves * 64) void k_gateup_few(GateUpFewArgs a) {
  __shared__ uint4 lds4[(kSignTab + kGridTab) / 16 + kFewTok * kXsStride];
  uint8_t* stab = (uint8_t*)lds4;                  // 32 KB
  uint8_t* gtab = stab + kSignTab;                 // 64 KB
  uint4* xs = lds4 + (kSignTab + kGridTab) / 16;  // 34 KB
  const int item = (int)blockIdx.y;
  if (item >= a.n_items[0]) return;
  const int e = load_scalar_i32(a.items, 3 * item);
  const int row0 = load_scalar_i32(a.items, 3 * item + 1);
  const int nrows = load_scalar_i32(a.items, 3 * item + 2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f0 = blockIdx.x * kFewFeat + 2 * w;
  // grid bytes (table build), then the wave's four rows
  uint2 gb = make_uint2(0, 0);
  if (tid < 256) gb = *(const uint2*)(a.grid + 8 * tid);
  const Iq2Off off = iq2_offsets(lane);
  Iq2Seg sg[2], su[2];
#pragma unroll
  for (int r = 0; r < 2; r++) {
    const size_t rowi = (size_t)e * kI + f0 + r;
    iq2_load((const uint32_t*)(a.gate + rowi * kRowIq2), 0, off, sg[r]);
    iq2_load((const uint32_t*)(a.up + rowi * kRowIq2), 0, off, su[r]);
  }
  if (tid < 256) store_copies(gtab, tid, grid_pairs(gb));
  else if (tid < 384) store_copies(stab, tid - 256, sign_masks(tid - 256));
  const uint32_t sh = ((lane >> 2) & 1) ? 0u : 2u;
  const uint32_t rep16 = (uint32_t)(lane & 15) << 4;
  const uint4* xl = xs + 8 * lane + (lane >> 1);  // chunk 8 lane
  for (int j0 = 0; j0 < nrows; j0 += kFewTok) {
    const int nt = min(kFewTok, nrows - j0);
    // an empty asm that "changes" the weight words, so that the decode's
    // table addresses (functions of them alone) are not hoisted out of the
    // pass loop: kept live across it they would not fit the registers
#pragma unroll
    for (int r = 0; r < 2; r++) {
      asm volatile("" : "+v"(sg[r].w0), "+v"(sg[r].w1), "+v"(sg[r].w2), "+v"(sg[r].w3),
                   "+v"(sg[r].w4), "+v"(sg[r].dw));
      asm volatile("" : "+v"(su[r].w0), "+v"(su[r].w1), "+v"(su[r].w2), "+v"(su[r].w3),
                   "+v"(su[r].w4), "+v"(su[r].dw));
    }
    if (j0 > 0) __syncthreads();  // every wave is done with the last pass's x
    // x of the pass's tokens: chunk q = tid + 1024 i of the kFewTok tokens'
    // chunks, token jj = q / kXsTok (wave-uniform)
#pragma unroll
    for (int i = 0; i < kFewTok * kXsTok / (kFewWaves * 64); i++) {
      const int q = tid + kFewWaves * 64 * i, jj = q / kXsTok, c = q % kXsTok;
      if (jj < nt) {
        const int tok = load_scalar_i32(a.perm, row0 + j0 + jj) / 6;
        xs[jj * kXsStride + c + (c >> 4)] = ((const uint4*)(a.x + (size_t)tok * kH))[c];
      }
    }
    __syncthreads();
    float acc[4][kFewTok];  // rows: gate f0, gate f0+1, up f0, up f0+1
    iq2_dot16_multi<kFewTok>(sg[0], sh, xl, gtab, stab, rep16, nt, acc[0]);
    iq2_dot16_multi<kFewTok>(sg[1], sh, xl, gtab, stab, rep16, nt, acc[1]);
    iq2_dot16_multi<kFewTok>(su[0], sh, xl, gtab, stab, rep16, nt, acc[2]);
    iq2_dot16_multi<kFewTok>(su[1], sh, xl, gtab, stab, rep16, nt, acc[3]);
    // two tokens per reduction: v = gate (f0, j), (f0+1, j), (f0, j+1),
    // (f0+1, j+1), then the same four up totals; lane 16 rho holds the gate
    // total of v[c[rho]] (c = {0, 2, 1, 3}), its up total 8 lanes further on
#pragma unroll
    for (int jp = 0; jp < kFewTok; jp += 2) {
      if (jp >= nt) continue;
      float v[8] = {acc[0][jp], acc[1][jp], acc[0][jp + 1], acc[1][jp + 1],
                    acc[2][jp], acc[3][jp], acc[2][jp + 1], acc[3][jp + 1]};
      if (jp + 1 >= nt) v[2] = v[3] = v[6] = v[7] = 0.0f;
      const float tot = reduce8(v);
      const float upv = dpp_f32<0x128>(tot);
      const int rho = lane >> 4;
      const int ci = (rho == 1) ? 2 : (rho == 2) ? 1 : rho;
      const int jj = jp + (ci >> 1);
      if ((lane & 15) == 0 && jj < nt) {
        const int pair = a.perm[row0 + j0 + jj];
        a.h[(size_t)pair * kI + f0 + (ci & 1)] = silu(tot) * upv;
      }
    }
  }
}

// down + weighted combine (+ residual) for one token.
// Grid (H / kDnBlockRows, T), 12 waves: wave w handles routed slot k = w / 2
// for kDnRows rows (w odd: the second half of the workgroup's 16 rows), two
// rows per step: lanes 0-31 take the even row, lanes 32-63 the odd one.
// Each lane requests its slot's SwiGLU values before the weights (the vector
// memory path of a compute unit returns data in request order, so h must not
// queue behind weights): straight from global memory (up to 4 tokens, and
// whenever a shared expert rides along as the seventh slot), or with STAGE
// (more than 4 tokens, no seventh slot) from LDS, where the workgroup copies
// the token's six vectors (48 KB) before the weights are requested.
// Lane 32u + L (L < 32), b = L >> 2, hq = (L >> 1) & 1, p = L & 1, covers
// the 64 columns i = 256b + 128hq + 32s + 16p + l (s < 4, l < 16) of its
// row: their 2-bit codes are exactly the 16 bytes qs[32hq + 16p .. +15] of
// block b (one 16-byte load), their sub-blocks are j = 8hq + 2s + p (scale
// bytes 8hq + p + 2s, inside the 8 bytes at 8hq), and d, dmin sit at byte 80:
// three loads per lane serve two rows.  The lane's 64 SwiGLU values become
// 16-bit fixed point with one scale, h_i ~= S n_i,
// n_i = round(32767 h_i / max|h|) (relative error below 2^-16 of the chunk
// maximum; every later product is exact); lanes L and L + 32 need the same
// values, so each reads and converts 32 of them and the pair swaps the
// results (and their partial maxima) with v_permlane32_swap:
//   nr[8s + q] = (n[16s + 2q], n[16s + 2q + 1]) as int16 pairs,
//   xn[s] = sum_l n[16s + l]   (for the min term).
// The h vectors sit in LDS as 16-byte chunks; chunk G of a slot (G = f / 4
// for value f) is stored at G ^ ((G >> 6) & 3) ^ (((G >> 5) & 1) << 3), so
// that the 16 lanes one 16-byte LDS read serves hit 16 distinct bank groups.
constexpr int kDnBlockRows = 2 * kDnRows;  // 16 output rows per workgroup
constexpr int kDnThreads = 12 * 64;
constexpr int kDnThreadsSh = 14 * 64;      // with the shared expert as a seventh slot

// The workgroup's 16 rows of a Q8_0 shared expert's down, as the seventh slot
// (two more waves): partial sums of rows row0 + 2m + u, m < 4, in pr (the
// reduce4x2 layout), from the token's shared SwiGLU row sh_h, read from
// global memory by each lane (64 values) ahead of its weights.
// Defined with the shared-expert kernels (ffn_shared.hip).
__device__ void shared_down_slot(const float4* sh_h, const uint8_t* sh_down, int row0, int lane,
                                 float* pr);

__device__ inline int dn_chunk(int G) {
  return G ^ ((G >> 6) & 3) ^ (((G >> 5) & 1) << 3);
}

// Sums over the 32 lanes of each wave half of four per-lane values at once
// (value m of half u is row 2m + u of the wave).  Lane L ends up holding the
// total of m = (rho & 1) + 2 * ((L >> 3) & 1), u = rho >> 1, rho = L >> 4;
// every lane of an aligned group of 8 holds the same total.
__device__ inline float reduce4x2(const float* v) {
  float w[2];
#pragma unroll
  for (int q = 0; q < 2; q++) {
    // rows of 16: row 0 <- v[2q] (half 0), row 1 <- v[2q+1] (half 0),
    // row 2 <- v[2q] (half 1), row 3 <- v[2q+1] (half 1)
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[2 * q]),
                                              __float_as_uint(v[2 * q + 1]), false, false);
    w[q] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  // within rows of 16: lanes 0-7 <- w[0], lanes 8-15 <- w[1]
  const bool up8 = (threadIdx.x & 8) != 0;
  const float t = up8 ? w[0] : w[1];
  float z = (up8 ? w[1] : w[0]) + dpp_f32<0x128>(t);  // row_ror:8
  z += dpp_f32<0xB1>(z);
  z += dpp_f32<0x4E>(z);
  z += dpp_f32<0x141>(z);
  return z;
}

// SH: a Q8_0 shared expert rides along as a seventh slot (waves 12 and 13,
// reading its SwiGLU row sh_h from global memory; only without STAGE),
// added unscaled.
template <bool SH, bool STAGE>
__global__ __launch_bounds__(SH ? kDnThreadsSh : kDnThreads) void k_down_q2k_b1(
    const float* __restrict__ h, const uint8_t* __restrict__ down,
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int E,
    float* __restrict__ out, float* __restrict__ residual, uint32_t* status,
    const float* __restrict__ sh_h, const uint8_t* __restrict__ sh_down) {
  constexpr int R = kDnRows;
  constexpr int kSlots = SH ? 7 : 6;
  static_assert(R == 8, "four steps of two rows per wave");
  __shared__ float part[kSlots][kDnBlockRows];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int k = w >> 1, rh = w & 1;
  const bool shw = SH && k == 6;  // a shared-slot wave
  const int u = lane >> 5, L = lane & 31, b = L >> 2, hq = (L >> 1) & 1, p = L & 1;
  // token t = blockIdx.y
  const int tok = blockIdx.y;
  h += (size_t)tok * 6 * kI;
  if (SH) sh_h += (size_t)tok * kI;
  ids += 6 * tok;
  wts += 6 * tok;
  if (out) out += (size_t)tok * kH;
  if (residual) residual += (size_t)tok * kH;
  // the expert id and gate first: the weight addresses wait for the id
  int e = shw ? 0 : load_scalar_i32(ids, k);
  const float wk = shw ? 1.0f : __int_as_float(load_scalar_i32((const int32_t*)wts, k));
  // the residual rows this workgroup adds to, requested before anything else:
  // read at the end, their round trip came after all the arithmetic
  float res_in = 0.0f;
  if (residual && tid < kDnBlockRows) res_in = residual[blockIdx.x * kDnBlockRows + tid];
  // Lane chunk order of the 64 values a lane consumes: chunk G0 + 8s + m4 of
  // its slot (16 bytes each) holds values 16s + 4m4 .. +3.
  const int G0 = 64 * b + 32 * hq + 4 * p;
  float hv[32];
  auto take = [&](int s, int m4, float4 q) {
    hv[16 * s + 4 * m4 + 0] = q.x;
    hv[16 * s + 4 * m4 + 1] = q.y;
    hv[16 * s + 4 * m4 + 2] = q.z;
    hv[16 * s + 4 * m4 + 3] = q.w;
  };
  static_assert(!(SH && STAGE), "the shared slot reads its row directly");
  // STAGE (many tokens): the six SwiGLU vectors are copied into LDS once per
  // workgroup and the weights requested after that barrier; at 8 and 12
  // tokens that took about 1-2% less time than per-wave reads, which read h
  // twice as often from L2.
  __shared__ float4 hs[STAGE ? 6 * kI / 4 : 1];
  if constexpr (STAGE) {
    static_assert(6 * kI / 4 == 4 * kDnThreads, "four h chunks per thread");
    float4 hc[4];
#pragma unroll
    for (int q = 0; q < 4; q++) hc[q] = ((const float4*)h)[tid + kDnThreads * q];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int G = tid + kDnThreads * q;
      hs[(G & ~511) | dn_chunk(G & 511)] = hc[q];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else if (!shw) {
    // 1. half of this lane's 64 values of slot k, requested ahead of the
    // weights: the two wave halves cover the same columns, so the lower half
    // reads and converts values 0-31 (s = 0, 1) and the upper half 32-63
    // (s = 2, 3), and they exchange the fixed-point results
    const float4* hk = (const float4*)h + 512 * k;
#pragma unroll
    for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
      for (int m4 = 0; m4 < 4; m4++) take(s2, m4, hk[G0 + 8 * (2 * u + s2) + m4]);
  }
  float pr[R / 2];
  bool bad_id = false;
  if (shw) {
    shared_down_slot((const float4*)sh_h, sh_down, blockIdx.x * kDnBlockRows + rh * R, lane, pr);
  } else {
  // 2. this wave's weights, requested behind its h
  bad_id = e < 0 || e >= E;
  e = bad_id ? 0 : e;
  const int row0 = blockIdx.x * kDnBlockRows + rh * R;  // output rows of token tok
  const uint8_t* base = down + ((size_t)e * kH + row0 + u) * kRowQ2k + b * kQ2kBytes;
  uint4 cv[R / 2];
  uint2 sc[R / 2];
  uint32_t dd[R / 2];
#pragma unroll
  for (int m = 0; m < R / 2; m++) {
    const uint8_t* blk = base + 2 * m * kRowQ2k;
    cv[m] = *(const uint4*)(blk + 16 + 32 * hq + 16 * p);
    sc[m] = *(const uint2*)(blk + 8 * hq);
    dd[m] = *(const uint32_t*)(blk + 80);
  }
  if constexpr (!STAGE) __builtin_amdgcn_sched_barrier(0);  // every load ahead of the arithmetic
  // 3. this lane's 64 values of slot k, as 16-bit fixed point (each wave
  // half takes 32 of them, as above)
  if constexpr (STAGE) {
#pragma unroll
    for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
      for (int m4 = 0; m4 < 4; m4++)
        take(s2, m4, hs[512 * k + dn_chunk(G0 + 8 * (2 * u + s2) + m4)]);
  }
  uint32_t nr[32];
  int xn[4];
  float S;
  {
    // the half's 32 values: the largest magnitude over both halves (the
    // pair of lanes L and L + 32 swap their partial maxima), then the
    // fixed point of the half's values and of its two sub-block sums, which
    // the lane pair swaps so that both hold all 64
    AbsMax am;
#pragma unroll
    for (int i = 0; i < 32; i++) am.add(hv[i]);
    {
      const auto rs = __builtin_amdgcn_permlane32_swap((uint32_t)am.smax, (uint32_t)am.smax, false, false);
      const auto ru = __builtin_amdgcn_permlane32_swap(am.umax, am.umax, false, false);
      am.smax = max((int)rs[0], (int)rs[1]);
      am.umax = max((uint32_t)ru[0], (uint32_t)ru[1]);
    }
    bool nonfinite;
    const float mx = am.value(nonfinite);
    const float inv = mx > 0.0f ? 1.0f / mx : 0.0f;
    uint32_t own[16];
#pragma unroll
    for (int q = 0; q < 16; q++)
      own[q] = (uint32_t)__builtin_bit_cast(
          int, __builtin_amdgcn_cvt_pknorm_i16(hv[2 * q] * inv, hv[2 * q + 1] * inv));
#pragma unroll
    for (int q = 0; q < 16; q++) {  // lower half's values (s = 0, 1), then the upper half's
      const auto r = __builtin_amdgcn_permlane32_swap(own[q], own[q], false, false);
      nr[q] = (uint32_t)r[0];
      nr[16 + q] = (uint32_t)r[1];
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
      int t = 0;
#pragma unroll
      for (int q = 0; q < 8; q++) t = sdot2(nr[8 * s + q], 0x00010001u, t);
      xn[s] = t;
    }
    // a NaN or infinite SwiGLU value makes every row of the slot NaN, as
    // the exact products would (the fixed point cannot carry it)
    S = nonfinite ? __builtin_nanf("") : mx * (1.0f / 32767.0f);
  }
  // 4. the rows
  const float wS = wk * S;
  const uint32_t ssel = (uint32_t)p | ((uint32_t)(p + 2) << 8) | ((uint32_t)(p + 4) << 16) |
                        ((uint32_t)(p + 6) << 24);
#pragma unroll
  for (int m = 0; m < R / 2; m++) {
    // the code bytes l = 2q, 2q + 1 in the two 16-bit halves
    uint32_t P[8];
    const uint32_t cw[4] = {cv[m].x, cv[m].y, cv[m].z, cv[m].w};
#pragma unroll
    for (int q = 0; q < 8; q++) P[q] = vperm(0u, cw[q >> 1], (q & 1) ? 0x0C030C02u : 0x0C010C00u);
    const uint32_t S4 = vperm(sc[m].y, sc[m].x, ssel);  // scale | min << 4 of sub-block s
    int A = 0, B = 0;
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const uint32_t mk = 0x00030003u << (2 * s);
      int t = 0;
#pragma unroll
      for (int q = 0; q < 8; q++) t = sdot2(P[q] & mk, nr[8 * s + q], t);
      t >>= 2 * s;  // codes were read in place, i.e. times 4^s; exact
      // |t| <= 3 * 16 * 32767 and |xn| <= 16 * 32767 fit 24 bits: full-rate
      // 24-bit multiply-adds, exact
      A = __mul24((int)((S4 >> (8 * s)) & 0xFu), t) + A;
      B = __mul24((int)((S4 >> (8 * s + 4)) & 0xFu), xn[s]) + B;
    }
    const float d = f16_bits_to_f32(dd[m] & 0xFFFFu), dmin = f16_bits_to_f32(dd[m] >> 16);
    pr[m] = wS * fmaf(-dmin, (float)B, d * (float)A);
  }
  }  // routed slot
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
    if (SH) acc += part[kSlots - 1][tid];
    const int row = blockIdx.x * kDnBlockRows + tid;
    if (residual) residual[row] = res_in + acc;
    else out[row] = acc;
  }
  if (bad_id && lane == 0 && blockIdx.x == 0 && rh == 0) raise_fault(status, DS4MOE_FAULT_BAD_ID);
}

}  // namespace ds4
