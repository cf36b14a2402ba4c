// grouped.hip -- several tokens per expert: token->expert permutation and the
// grouped MFMA expert FFN (batched decode and prefill), gfx950.
//
// Method: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed, sections
// "MoE FFN 部の中身" (E(x) = W_down(SiLU(W_gate x) * W_up x), weighted sum,
// always-on shared expert) and "プリフィルとデコードで何が違うか" (with many
// tokens the union of selected experts approaches all of them, so the work is
// a grouped matrix product per expert).  Formats: DS4C2 =
// qiita.com/yoshiyakato/items/4678be0e7860ddb444ec, sections 3 and 4; FLOW
// quantisation table (Q8_0).
//
// Rows: the (token, slot) pairs sorted by expert occupy rows [0, T*K) (row i
// is pair perm[i]); the shared expert's rows are [T*K, T*K + T) (token order).
// Work items (expert, first row, row count <= 64) are listed by the
// permutation kernel; a grouped kernel block takes one item and 64 output
// features.
//
// Exactness: MFMA operands are exact.  IQ2_XXS gate/up (f16 MFMA
// 16x16x32): A = x in binary16 (exact for the bf16 inputs within the
// binary16 range), B = grid value * sign * (2s + 1) (an integer, exact); the
// block scale d rescales the fp32 accumulators.  Other gate/up formats (bf16
// MFMA 16x16x32): A = x as given, B = the grid value * sign or the Q8_0 code;
// each 32-column group's scale multiplies that group's MFMA result.  down (f16 MFMA 16x16x16,
// one 16-value Q2_K sub-block per step): A = the SwiGLU output split as
// f16 hi + lo (relative error < 2^-21), B = the 2-bit code masked in place in
// a 16-bit lane, i.e. the binary16 subnormal 4^s q 2^-24; the sub-block factor
// d*sc*4^-s*2^24 multiplies each step's result; the mins enter through a
// second MFMA on per-sub-block sums of h against the min nibbles.  Sums are
// fp32 throughout.
#include <type_traits>

#include "dev_common.h"

namespace ds4 {

constexpr int kMC = 64;   // rows (pairs) per work item
// Routed work items of calls with at most kSmallPieceMaxT tokens are cut into
// 16-row pieces, so that every item runs in the small-item kernels (one
// 16-row tile, many workgroups per expert) instead of a few 64-row items
// setting the pace; larger calls use 64-row pieces (each weight decoded once
// per 64 rows).
constexpr int kSmallPieceMaxT = 64;
__host__ __device__ inline int item_rows(int T) { return T <= kSmallPieceMaxT ? 16 : kMC; }
constexpr int kNT = 64;   // output features per block (16 per wave)
constexpr int kGW = 8;             // pipelined IQ2_XXS gate/up: waves per block
constexpr int kGNF = 16 * kGW;     // and features per block
constexpr int kGStage = 128;       // and K columns per stage
constexpr int kDW = 8;             // pipelined Q2_K down: waves per block
constexpr int kDNF = 16 * kDW;     // and output features per block
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void k_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                                  int32_t* offsets, int32_t* perm, int32_t* inv,
                                                  uint32_t* status, int T, int with_shared,
                                                  int32_t* items, int32_t* n_items);

// Work list: items (e, row0, nrows) for every expert with pairs (pieces of
// item_rows(T) rows), then the shared expert's rows (e == E, 64-row pieces).
// Items of at most 16 rows (with 64-row pieces an expert's last piece) come
// first, in ascending expert order, so that a kernel specialised for one
// 16-row tile can take them; n_items[0] is the number of items, n_items[1]
// the number of those small ones.  One wave of 64 threads, four experts per
// lane, prefix sums over the lanes.
__device__ inline int wave_prefix_excl(int v, int& total) {
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if ((int)(threadIdx.x & 63) >= d) incl += u;
  }
  total = __shfl(incl, 63);
  return incl - v;
}

// The work list by one wave (lane = threadIdx.x mod 64), built inside
// k_permute from its LDS copies of the counts and offsets.
__device__ void make_items_wave(const int32_t* counts, const int32_t* offsets, int E, int TK, int T,
                                int with_shared, int32_t* items, int32_t* n_items) {
  const int lane = threadIdx.x & 63;
  const int P = item_rows(T);
  int cnt[4], nsm = 0, nlg = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = 4 * lane + j;
    cnt[j] = e < E ? counts[e] : 0;
    const int full = cnt[j] / P, rem = cnt[j] % P;
    nsm += (P <= 16 ? full : 0) + ((rem > 0 && rem <= 16) ? 1 : 0);
    nlg += (P > 16 ? full : 0) + (rem > 16 ? 1 : 0);
  }
  int small_total, large_total;
  int ps = wave_prefix_excl(nsm, small_total);
  int pl = small_total + wave_prefix_excl(nlg, large_total);
  auto put = [&](int i, int e, int r0, int nr) {
    items[3 * i] = e;
    items[3 * i + 1] = r0;
    items[3 * i + 2] = nr;
  };
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int e = 4 * lane + j;
    for (int m0 = 0; m0 < cnt[j]; m0 += P) {
      const int nr = min(P, cnt[j] - m0);
      if (nr <= 16) put(ps++, e, offsets[e] + m0, nr);
      else put(pl++, e, offsets[e] + m0, nr);
    }
  }
  const int routed = small_total + large_total;
  const int ns = with_shared ? (T + kMC - 1) / kMC : 0;
  for (int i = lane; i < ns; i += 64) put(routed + i, E, TK + kMC * i, min(kMC, T - kMC * i));
  if (lane == 0) {
    n_items[0] = routed + ns;
    n_items[1] = small_total;
  }
}

// Work list of the shared expert alone (its rows T*K .. T*K+T-1), for calls
// whose routed experts take the few-token path.
__global__ void k_make_shared_items(int E, int TK, int T, int32_t* items, int32_t* n_items) {
  const int i = threadIdx.x, ns = (T + kMC - 1) / kMC;
  for (int j = i; j < ns; j += blockDim.x) {
    items[3 * j] = E;
    items[3 * j + 1] = TK + kMC * j;
    items[3 * j + 2] = min(kMC, T - kMC * j);
  }
  if (i == 0) {
    n_items[0] = ns;
    n_items[1] = 0;
  }
}

// dst[t][c] += shared expert output of token t: y[T*K + t][c], or the sum of
// its K shares part[z][t][c] taken in z order.
__global__ void k_add_shared(const float* y, const float* part, int ks, int TK, int T, int H,
                             float* dst) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T * H) return;
  float v;
  if (ks == 1) {
    v = y[(size_t)TK * H + idx];
  } else {
    v = 0.0f;
    for (int z = 0; z < ks; z++) v += part[(size_t)z * T * H + idx];
  }
  dst[idx] += v;
}

inline int max_items(int E, int TK, int T, bool shared) {
  const int P = item_rows(T);
  return E + (TK + P - 1) / P + (shared ? (T + kMC - 1) / kMC : 0);
}
// The most work items a call of at most T tokens lists (16-row pieces can
// list more items at 64 tokens than 64-row pieces at 65): the workspace size,
// which so stays monotone in the token count.
inline int max_items_upto(int E, int K, int T) {
  const int t16 = T < kSmallPieceMaxT ? T : kSmallPieceMaxT;
  const int m16 = max_items(E, t16 * K, t16, true), m = max_items(E, T * K, T, true);
  return m16 > m ? m16 : m;
}
// Grid rows of the small-item kernels: at most one small item per expert
// with 64-row pieces; with 16-row pieces every routed item is small.
inline int max_small_items(int E, int TK, int T) {
  const int m = item_rows(T) <= 16 ? E + (TK + 15) / 16 : E;
  return m < TK ? m : TK;
}

struct GroupArgs {
  int H, I, E, K, T;
  const uint16_t* x;        // [T][H] bf16
  const uint16_t* x16;      // [T][H] the same in binary16 (IQ2_XXS gate/up)
  const int32_t* perm;      // [T*K]
  const int32_t* items;     // [n][3]
  const int32_t* n_items;
  const uint8_t *gate, *up, *down;
  int qt_g, qt_u, qt_d;
  const uint8_t *sh_gate, *sh_up, *sh_down;
  int sh_qt_g, sh_qt_u, sh_qt_d, sh_I;
  const uint8_t* grid;
  int8_t* xrexp;            // [T*K + 64][4] x16 = x * 2^e per token: word j packs e of sorted
                            // rows j .. j + 3 (byte r: row j + r), one aligned load per lane
  uint16_t* hh;             // [T*K + T][I] SwiGLU rows times 2^hexp, binary16 high part
  uint16_t* hl;             // [T*K + T][I] binary16 low part (h - hi, rounded)
  uint16_t* hsh;            // [T*K + T][I/16] sums of 16 consecutive features, high part
  uint16_t* hsl;            // [T*K + T][I/16] low part
  int8_t* hexp;             // [T*K + T][I/64] the exponent of each row's 64-feature range
  float* y;                 // [T*K + T][H] fp32
  uint32_t* status;
  // K split of the shared expert's kernels (few-token calls): partial sums
  // [split][T][2*I] (gate, up) then [split][T][H] (down), reduced in a fixed order
  int ksplit_g, ksplit_d;
  float* part;
  // > 0: the grid rows cover only the shared expert's work items, the last
  // sh_tail of the list (launches of kernels that see shared rows only)
  int sh_tail;
};

// The work item of grid row blockIdx.y.
__device__ inline int grid_item(const GroupArgs& a) {
  return a.sh_tail > 0 ? a.n_items[0] - a.sh_tail + (int)blockIdx.y : (int)blockIdx.y;
}

__device__ inline int row_token(const GroupArgs& a, int row) {
  return row < a.T * a.K ? a.perm[row] / a.K : row - a.T * a.K;
}

// The power-of-two exponent e that brings a largest magnitude M into
// [2^top, 2^(top+1)); 0 for M = 0 and for NaN or infinite values (they then
// propagate as they are).  |e| <= 120.
__device__ inline int pow2_exponent(float M, bool bad, int top) {
  if (bad || !(M > 0.0f)) return 0;
  int k;
  (void)frexpf(M, &k);  // M = f 2^k, 1/2 <= f < 1
  return min(max(top - k + 1, -120), 120);
}

// AbsMax over the lanes of a wave (every lane receives the result).
__device__ inline AbsMax wave_absmax(AbsMax v) {
  AbsMax r;
  r.smax = (int)(wave_max_u32((uint32_t)v.smax ^ 0x80000000u) ^ 0x80000000u);
  r.umax = wave_max_u32(v.umax);
  return r;
}

// SwiGLU epilogue of the grouped gate/up kernels.  Lane (column n = lane%16,
// quarter q) holds rows 4q + r of each 16-row tile.  The down kernels take h
// as binary16 high + low parts (relative error < 2^-21) and, for the Q2_K
// min term, the sum of each 16 consecutive features (a wave's tile) split
// the same way; the sum runs over the 16 lanes of a DPP row in a fixed order.
// So that any magnitude fits binary16, the stored values are h * 2^e with
// one exponent per work item and feature tile (features n0 .. n0 + nf - 1):
// 0 while the largest |h| of the tile, over every wave of the block, stays
// below 2^11 (the sums of 16 then stay below 2^15), else the exponent that
// brings it into [2^10, 2^11); scaling by a power of two is exact.  Each
// wave stores its rows with e = 0 at once and, in the rare case e != 0,
// again once the block has agreed on e; e is written for each row and
// 64-feature range of the tile.  xe (binary16 x): the accumulators of rows
// 16 mt + 4q + r are in units of 2^xe[mt][r], the x exponent of the row's
// token (loaded by the caller ahead of its main loop), undone first;
// nullptr otherwise.  red: 32 words of the caller's LDS that no wave touches
// once the caller's last barrier has passed (its staging buffers, free after
// the main loop: a block-wide array of its own here would push the iq2
// kernels past 80 KB and halve their occupancy).  Every thread of the block
// must call it.
template <int MT = 4>
__device__ inline void swiglu_store(const GroupArgs& a, int row0, int nrows, int mtiles, int n,
                                    int q, const f32x4_t* accg, const f32x4_t* accu, int n0,
                                    int nf, const uint32_t* xe, uint32_t* red) {
  float v[MT][4];
  AbsMax am;
  auto store = [&](int e) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      if (mt >= mtiles) break;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = 16 * mt + 4 * q + r;
        const float vs = ldexpf(v[mt][r], e);
        const uint32_t hi = f32_to_f16_bits(vs);
        const uint32_t lo = f32_to_f16_bits(vs - f16_bits_to_f32(hi));
        float sum = vs;
        sum += dpp_f32<0xB1>(sum);
        sum += dpp_f32<0x4E>(sum);
        sum += dpp_f32<0x141>(sum);
        sum += dpp_f32<0x140>(sum);
        if (m < nrows) {
          const size_t row = (size_t)(row0 + m);
          a.hh[row * a.I + n] = (uint16_t)hi;
          a.hl[row * a.I + n] = (uint16_t)lo;
          if ((n & 15) == 0) {
            const uint32_t shi = f32_to_f16_bits(sum);
            a.hsh[row * (a.I / 16) + n / 16] = (uint16_t)shi;
            a.hsl[row * (a.I / 16) + n / 16] = (uint16_t)f32_to_f16_bits(sum - f16_bits_to_f32(shi));
          }
        }
      }
    }
  };
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = 16 * mt + 4 * q + r;
      const bool live = mt < mtiles && m < nrows;
      float g = accg[mt][r], u = accu[mt][r];
      if (xe) {
        const int ex = (int8_t)(xe[mt] >> (8 * r));
        g = ldexpf(g, -ex);
        u = ldexpf(u, -ex);
      }
      v[mt][r] = live ? silu(g) * u : 0.0f;
      if (live) am.add(v[mt][r]);
    }
  store(0);
  am = wave_absmax(am);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) {
    red[w] = (uint32_t)am.smax;
    red[16 + w] = am.umax;
  }
  __syncthreads();
  AbsMax bm;
  for (int i = 0; i < nw; i++) {
    bm.smax = max(bm.smax, (int)red[i]);
    bm.umax = max(bm.umax, red[16 + i]);
  }
  bool bad;
  const float M = bm.value(bad);
  const int e = M < 2048.0f ? 0 : pow2_exponent(M, bad, 10);
  if ((int)threadIdx.x < nrows * (nf / 64)) {
    const int m = threadIdx.x / (nf / 64), rg = threadIdx.x % (nf / 64);
    a.hexp[(size_t)(row0 + m) * (a.I / 64) + n0 / 64 + rg] = (int8_t)e;
  }
  if (e != 0) store(e);  // the same lanes rewrite the same addresses
}

// The x exponents of rows row0 + 16 mt + 4q .. +3 (mt < MT), for
// swiglu_store; rows past the item read padding and are never used.
template <int MT>
__device__ inline void load_row_xexp(const GroupArgs& a, int row0, int q, uint32_t* xe) {
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
    xe[mt] = *(const uint32_t*)(a.xrexp + 4 * (size_t)(row0 + 16 * mt + 4 * q));
}

// 8 bytes at a 2-byte-aligned address (Q8_0 codes).
__device__ inline uint2 load8_a2(const uint8_t* p) {
  const uint16_t* q = (const uint16_t*)p;
  return make_uint2((uint32_t)q[0] | ((uint32_t)q[1] << 16), (uint32_t)q[2] | ((uint32_t)q[3] << 16));
}

// four signed bytes -> two bf16 pairs (exact: |c| <= 127)
__device__ inline void i8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  float f0 = (float)(int8_t)(w & 0xFF), f1 = (float)(int8_t)((w >> 8) & 0xFF);
  float f2 = (float)(int8_t)((w >> 16) & 0xFF), f3 = (float)(int8_t)(w >> 24);
  lo = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
  hi = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xFFFF0000u);
}
__device__ inline void i8x4_to_f16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = f32_to_f16_bits((float)(int8_t)(w & 0xFF)) | (f32_to_f16_bits((float)(int8_t)((w >> 8) & 0xFF)) << 16);
  hi = f32_to_f16_bits((float)(int8_t)((w >> 16) & 0xFF)) | (f32_to_f16_bits((float)(int8_t)(w >> 24)) << 16);
}

// IQ2_XXS grid / sign tables replicated 8x (see ffn_b1.hip), built by 256 threads.
__device__ inline void build_tables8_256(const uint8_t* grid, uint4* gt8, uint4* mt8) {
  const int t = threadIdx.x;
  {
    const uint8_t* g = grid + 8 * t;
    uint32_t w[4];
    for (int m = 0; m < 4; m++) {
      uint32_t lo = __float_as_uint((float)g[2 * m]) >> 16;
      uint32_t hi = __float_as_uint((float)g[2 * m + 1]) >> 16;
      w[m] = lo | (hi << 16);
    }
    const uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
    for (int q = 0; q < 8; q++) gt8[8 * t + q] = v;
  }
  if (t < 128) {
    uint32_t s8 = (uint32_t)t | ((uint32_t)(__popc(t) & 1) << 7);
    uint32_t w[4];
    for (int m = 0; m < 4; m++)
      w[m] = (((s8 >> (2 * m)) & 1u) << 15) | (((s8 >> (2 * m + 1)) & 1u) << 31);
    const uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
    for (int q = 0; q < 8; q++) mt8[8 * t + q] = v;
  }
}

// B fragment (8 values) of a gate/up row for one 32-column group, plus the
// group scale.  IQ2_XXS: lane sub-vector q of group g of the 256-block at blk.
__device__ inline void iq2_bfrag(const uint8_t* blk, int g, int q, int rep, const uint4* gt8,
                                 const uint4* mt8, bf16x8_t& b, float& scale) {
  const uint8_t* gp = blk + 2 + 8 * g;
  uint32_t idx = gp[q];
  const uint16_t* sp = (const uint16_t*)(gp + 4);
  uint32_t sw = (uint32_t)sp[0] | ((uint32_t)sp[1] << 16);
  float d = f16_bits_to_f32((uint32_t)((const uint16_t*)blk)[0]);
  scale = d * (float)(2u * (sw >> 28) + 1u) * 0.125f;
  uint4 gv = gt8[8 * idx + rep];
  uint4 mv = mt8[8 * ((sw >> (7 * q)) & 0x7Fu) + rep];
  uint4 v = make_uint4(gv.x ^ mv.x, gv.y ^ mv.y, gv.z ^ mv.z, gv.w ^ mv.w);
  b = __builtin_bit_cast(bf16x8_t, v);
}
// Q8_0: 32-value block g (of the 256-column chunk at chunk), lane's 8 codes.
__device__ inline void q80_bfrag(const uint8_t* chunk, int g, int q, bf16x8_t& b, float& scale) {
  const uint8_t* bp = chunk + g * kQ80Bytes;
  scale = f16_bits_to_f32((uint32_t)((const uint16_t*)bp)[0]);
  uint2 c = load8_a2(bp + 2 + 8 * q);
  uint4 v;
  i8x4_to_bf16x4(c.x, v.x, v.y);
  i8x4_to_bf16x4(c.y, v.z, v.w);
  b = __builtin_bit_cast(bf16x8_t, v);
}

__host__ __device__ inline bool iq2_grouped_fast(const GroupArgs& a) {
  return a.qt_g == DS4MOE_IQ2_XXS && a.qt_u == DS4MOE_IQ2_XXS && a.I % kGNF == 0 && a.H % 512 == 0 &&
         (uintptr_t)a.grid % 8 == 0;
}

// The pipelined Q2_K down takes its rows from the pipelined IQ2_XXS gate/up,
// whose 128-feature tiles match its 128-column stages (one binary16 exponent
// per work item and stage).
__host__ __device__ inline bool q2k_grouped_fast(const GroupArgs& a) {
  return a.qt_d == DS4MOE_Q2_K && a.H % kDNF == 0 && a.I % 512 == 0 && a.I <= 8192 &&
         iq2_grouped_fast(a);
}

// The pipelined Q4_K down follows each 64-column chunk's binary16 exponent,
// so it takes the rows of any grouped gate/up kernel.
__host__ __device__ inline bool q4k_grouped_dn(const GroupArgs& a) {
  return a.qt_d == DS4MOE_Q4_K && a.H % kDNF == 0 && a.I % 512 == 0 && a.I <= 8192;
}

__host__ __device__ inline bool q80_shared_fast(const GroupArgs& a) {
  return a.sh_qt_g == DS4MOE_Q8_0 && a.sh_qt_u == DS4MOE_Q8_0 && a.sh_I % kGNF == 0 && a.H % 64 == 0;
}

// ---------------------------------------------------------------------------
// Q4_K experts (the mixed stacks' Q4 layers) on the grouped path.  Block:
// fp16 d, fp16 dmin, twelve bytes of 6-bit scales sc_j and mins m_j of the
// eight 32-column groups, 128 code bytes (byte 16 + 32c + l: column 64c + l
// in the low nibble, 64c + 32 + l in the high one); value = d sc_j q -
// dmin m_j.  A lane quarter q takes the 8 columns 32j + 8q .. +7 of group j:
// 8 consecutive code bytes, each in the low (even j) or high (odd j) nibble.
// Masked in place inside 16-bit lanes they are the binary16 subnormals
// q 2^-24 (low) or 16 q 2^-24 (high), exact, and form the f16 B fragment; the
// group factor d sc_j 2^24 (/16) multiplies that MFMA's result.  The mins
// need the sum of A over each group: gate/up take it from one more MFMA
// against a fragment of ones, down from the per-16-feature sums of h.
// ---------------------------------------------------------------------------
__device__ inline void q4k_scale_min(const uint4& hd, int j, int& sc, int& mn) {
  if (j < 4) {
    sc = (int)((hd.y >> (8 * j)) & 63u);
    mn = (int)((hd.z >> (8 * j)) & 63u);
  } else {
    const int k = 8 * (j - 4);
    sc = (int)(((hd.w >> k) & 15u) | (((hd.y >> (k + 6)) & 3u) << 4));
    mn = (int)(((hd.w >> (k + 4)) & 15u) | (((hd.z >> (k + 6)) & 3u) << 4));
  }
}

// the lane's 8 code bytes as four 16-bit-lane pairs (bytes 0,1 | 2,3 | 4,5 | 6,7)
__device__ inline uint4 q4k_pairs(uint2 c) {
  return make_uint4(vperm(0u, c.x, 0x0C010C00u), vperm(0u, c.x, 0x0C030C02u),
                    vperm(0u, c.y, 0x0C010C00u), vperm(0u, c.y, 0x0C030C02u));
}
__device__ inline f16x8_t q4k_frag(const uint4& p, bool high) {
  const uint32_t M = high ? 0x00F000F0u : 0x000F000Fu;
  return __builtin_bit_cast(f16x8_t, make_uint4(p.x & M, p.y & M, p.z & M, p.w & M));
}

__host__ __device__ inline bool q4k_grouped_gu(const GroupArgs& a) {
  return a.qt_g == DS4MOE_Q4_K && a.qt_u == DS4MOE_Q4_K;
}

// gate/up + SwiGLU for one work item and 64 intermediate features.
// Grid (ceil(Imax/64), max_items), 256 threads; wave w owns features
// n0 + 16w .. +15 (gate and up).  x tile staged in LDS per 128 columns with
// 16-byte chunk c of row m at slot c ^ (m & 15) (conflict-free A reads: the
// 16 lanes served together read 16 different bank groups).
__global__ __launch_bounds__(256) void k_grouped_gateup(GroupArgs a) {
  __shared__ uint4 xt[kMC * 16];
  __shared__ uint4 gt8[256 * 8];
  __shared__ uint4 mt8[128 * 8];
  __shared__ int tok[kMC];
  const int item = grid_item(a);
  if (item >= *a.n_items) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  const bool sh = e == a.E;
  // routed items with IQ2_XXS gate and up run in k_grouped_gateup_iq2, a
  // Q8_0 shared expert in k_grouped_gateup_q80
  if (!sh && (iq2_grouped_fast(a) || q4k_grouped_gu(a))) return;
  if (sh && q80_shared_fast(a)) return;
  const int I = sh ? a.sh_I : a.I;
  const int n0 = blockIdx.x * kNT;
  if (n0 >= I) return;
  const int qg = sh ? a.sh_qt_g : a.qt_g, qu = sh ? a.sh_qt_u : a.qt_u;
  const uint8_t* G = sh ? a.sh_gate : a.gate;
  const uint8_t* U = sh ? a.sh_up : a.up;
  const int ee = sh ? 0 : e;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4, rep = lane & 7;
  const int n = n0 + 16 * w + (lane & 15);
  const int nb = a.H / 256;  // 256-column chunks per row
  if (tid < kMC) tok[tid] = tid < nrows ? row_token(a, row0 + tid) : -1;
  if (qg == DS4MOE_IQ2_XXS || qu == DS4MOE_IQ2_XXS) build_tables8_256(a.grid, gt8, mt8);
  const size_t rowg = (size_t)ee * I + n;
  const int bbg = block_bytes(qg) * (256 / block_values(qg));  // bytes per 256 columns
  const int bbu = block_bytes(qu) * (256 / block_values(qu));
  const int mtiles = (nrows + 15) >> 4;
  f32x4_t accg[4], accu[4];
  for (int mt = 0; mt < 4; mt++) accg[mt] = accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int kh = 0; kh < 2 * nb; kh++) {
    const int kb = kh >> 1, goff = 4 * (kh & 1);
    for (int c = tid; c < kMC * 16; c += 256) {
      const int m = c >> 4, ch = c & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < nrows) v = ((const uint4*)(a.x + (size_t)tok[m] * a.H + 128 * kh))[ch];
      xt[m * 16 + (ch ^ (m & 15))] = v;
    }
    __syncthreads();
    const uint8_t* bg = G + (rowg * nb + kb) * bbg;
    const uint8_t* bu = U + (rowg * nb + kb) * bbu;
#pragma unroll 1
    for (int gi = 0; gi < 4; gi++) {
      const int g = goff + gi;
      bf16x8_t fg, fu;
      float sg, su;
      if (qg == DS4MOE_IQ2_XXS) iq2_bfrag(bg, g, q, rep, gt8, mt8, fg, sg);
      else q80_bfrag(bg, g, q, fg, sg);
      if (qu == DS4MOE_IQ2_XXS) iq2_bfrag(bu, g, q, rep, gt8, mt8, fu, su);
      else q80_bfrag(bu, g, q, fu, su);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        if (mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, xt[m * 16 + ((4 * gi + q) ^ (m & 15))]);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, fg, z, 0, 0, 0);
        f32x4_t tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, fu, z, 0, 0, 0);
        accg[mt] += sg * tg;
        accu[mt] += su * tu;
      }
    }
    __syncthreads();
  }
  swiglu_store(a, row0, nrows, mtiles, n, q, accg, accu, n0, kNT, nullptr, (uint32_t*)xt);
}

// ---------------------------------------------------------------------------
// gate/up for routed items with IQ2_XXS gate and up: software-pipelined.
// Grid (I/128, items), 512 threads; wave w owns features n0 + 16w .. +15
// (gate and up).  K runs in stages of 128 columns (half an IQ2_XXS block:
// four 32-column sub-blocks).  In a stage, lane quarter q takes sub-block q
// whole: its four 8-value groups are the B fragments of the stage's four
// MFMA steps (step j covers columns 32q + 8j .. +7 of the stage in quarter
// q; the A fragments are read in the same column order, and a sum over K
// does not depend on that order).  The sub-block factor 2s + 1 is then one
// number per lane and goes into B, in binary16:
//   B = grid * sign * (2s + 1)   (an integer of at most 2046 for grid values
//                                 up to 66, so exact; the format's are 8..43)
//   A = x in binary16 (converted once per call).
// The block scale d is shared by the four quarters of a row (one block per
// stage pair) and by the accumulator columns a lane holds (its own feature),
// so it is applied to the fp32 accumulators: they hold the sum divided by the
// current block's d and are rescaled by d_prev / d at each block start (one
// rounding per block), times d / 8 at the end.  A lane needs only its
// sub-block's 8 bytes (three aligned words when the block starts two bytes
// into a word) and the word holding d, so four stages of weights fit in a
// register ring: stage s + 3 is requested while stage s is multiplied, and
// x rows two stages ahead go through registers into a double-buffered LDS
// tile.  One barrier per stage.
struct Iq2Sub {
  uint32_t w0, w1, w2, dw;
};

// Sub-block q of stage s.  EVEN: block s >> 1 is even, so (block size 66)
// its bytes start two bytes into a word; the third word then ends inside
// the next block, which exists (an even number of blocks per row).
template <bool EVEN>
__device__ inline void iq2_sub_load(const uint8_t* __restrict__ row, int s, int q, Iq2Sub& o) {
  const int kb = s >> 1;
  const int start = kIq2Bytes * kb + 2 + 32 * (s & 1) + 8 * q;
  const uint32_t* p = (const uint32_t*)(row + (start & ~3));
  o.w0 = p[0];
  o.w1 = p[1];
  if (EVEN) o.w2 = p[2];
  o.dw = *(const uint32_t*)(row + ((kIq2Bytes * kb) & ~3));
}

// index word, sign/scale word, the block's d (1 when d is 0) and the B factor
// (2s + 1) twice in binary16 (0 when d is 0)
template <bool EVEN>
__device__ inline uint32_t iq2_sub_words(const Iq2Sub& o, uint32_t& idx, uint32_t& sgn, float& d) {
  idx = EVEN ? align_bytes(o.w1, o.w0, 2) : o.w0;
  sgn = EVEN ? align_bytes(o.w2, o.w1, 2) : o.w1;
  const float dv = f16_bits_to_f32(EVEN ? (o.dw & 0xFFFFu) : (o.dw >> 16));
  d = dv != 0.0f ? dv : 1.0f;
  const uint32_t h = f32_to_f16_bits((float)(2u * (sgn >> 28) + 1u));
  return dv != 0.0f ? h | (h << 16) : 0u;
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// group j of the lane's sub-block as the binary16 B fragment
__device__ inline f16x8_t iq2_sub_frag(uint32_t idx, uint32_t sgn, int j, uint32_t sc2,
                                       uint32_t rep16, const uint8_t* gtab, const uint8_t* stab) {
  const uint32_t gi = (idx >> (8 * j)) & 0xFFu;
  const uint32_t si = (sgn >> (7 * j)) & 0x7Fu;
  const uint4 gv = *(const uint4*)(gtab + ((gi << 7) | rep16));
  const uint4 mv = *(const uint4*)(stab + ((si << 7) | rep16));
  const f16x2_t c = __builtin_bit_cast(f16x2_t, sc2);
  const f16x2_t b0 = __builtin_bit_cast(f16x2_t, gv.x ^ mv.x) * c;
  const f16x2_t b1 = __builtin_bit_cast(f16x2_t, gv.y ^ mv.y) * c;
  const f16x2_t b2 = __builtin_bit_cast(f16x2_t, gv.z ^ mv.z) * c;
  const f16x2_t b3 = __builtin_bit_cast(f16x2_t, gv.w ^ mv.w) * c;
  return __builtin_bit_cast(
      f16x8_t, make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                          __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3)));
}

// the IQ2_XXS grid in binary16 (entry e, copy p at (e << 7) | (p << 4); gb =
// the 8 grid bytes of entry threadIdx.x) and the 128 sign patterns as masks
// of the binary16 sign bits
__device__ inline void build_tables8_f16(uint2 gb, uint4* gt8, uint4* mt8) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    uint32_t wv[4];
    for (int m = 0; m < 4; m++) {
      const uint32_t b2 = (m < 2 ? gb.x : gb.y) >> (16 * (m & 1));
      wv[m] = f32_to_f16_bits((float)(b2 & 0xFFu)) | (f32_to_f16_bits((float)((b2 >> 8) & 0xFFu)) << 16);
    }
    const uint4 v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    for (int j = 0; j < 8; j++) gt8[8 * tid + ((j + tid) & 7)] = v;
  } else if (tid < 384) {
    const int t = tid - 256;
    const uint32_t s8 = (uint32_t)t | ((uint32_t)(__popc(t) & 1) << 7);
    uint32_t wv[4];
    for (int m = 0; m < 4; m++)
      wv[m] = (((s8 >> (2 * m)) & 1u) << 15) | (((s8 >> (2 * m + 1)) & 1u) << 31);
    const uint4 v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    for (int j = 0; j < 8; j++) mt8[8 * t + ((j + t) & 7)] = v;
  }
}

// LDS of the IQ2_XXS gate/up bodies, 80 KB (two blocks per CU): the grid and
// sign tables (32 + 16 KB) and 32 KB of x tiles.
constexpr int kGuLds = (256 * 8 + 128 * 8) + 2048;  // uint4 units

// The body for items of up to 16 MT rows (MT = 4: the 64-row items after the
// small ones); item: its index in the work list, lds: kGuLds uint4.
template <int MT>
__device__ __attribute__((always_inline)) inline void gateup_iq2_body(const GroupArgs& a, int item,
                                                                     uint4* lds) {
  constexpr int kRows = 16 * MT;                           // x tile rows
  constexpr int kXC = kRows * 16;                          // 16-byte chunks of an x stage
  constexpr int kXJ = (kXC + kGW * 64 - 1) / (kGW * 64);  // chunks per thread
  static_assert(2 * kXC <= 2048, "x tiles fit the LDS area");
  uint4* gt8 = lds;                                   // 32 KB
  uint4* mt8 = lds + 256 * 8;                         // 16 KB
  uint4 (*xt)[kXC] = (uint4 (*)[kXC])(lds + 256 * 8 + 128 * 8);  // 2 x (MT x 4 KB)
  if (item >= a.n_items[0]) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  if (e >= a.E) return;  // shared-expert items run in k_grouped_gateup
  const int n0 = blockIdx.x * kGNF;
  if (n0 >= a.I) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  const int n = n0 + 16 * w + (lane & 15);
  const uint32_t rep16 = (uint32_t)(lane & 7) << 4;
  const int rowbytes = (a.H / 256) * kIq2Bytes;
  const uint8_t* grow = a.gate + ((size_t)e * a.I + n) * rowbytes;
  const uint8_t* urow = a.up + ((size_t)e * a.I + n) * rowbytes;
  const int nst = a.H / kGStage;  // a multiple of 4
  const int mtiles = (nrows + 15) >> 4;

  // x chunk c = tid + 512 j (mod the tile) -> row c >> 4, 16-byte column
  // chunk c & 15.  Every lane loads (rows past the item repeat row 0: their
  // results are never stored) and stores (threads past the tile store the
  // same chunk again), so no branch lets the compiler move a load down to
  // its store or hide it from the wait counts.  Plain vector values, so
  // that nothing goes through a private array.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  struct XV {
    u32x4_t v[kXJ];
  };
  // Vector memory returns in order, so the loads go out in the order they
  // are needed: the grid bytes and the tokens of this thread's x rows, the
  // weights of stages 0 and 1, x of stages 0 and 1, then the weights of
  // stage 2 (in the loop, as in the first stage, x then weights).
  const uint2 gb = *(const uint2*)(a.grid + 8 * (tid & 255));
  int xtok[kXJ];
#pragma unroll
  for (int j = 0; j < kXJ; j++) {
    const int m = ((tid + kGW * 64 * j) & (kXC - 1)) >> 4;
    xtok[j] = a.perm[row0 + (m < nrows ? m : 0)] / a.K;  // routed rows only
  }
  __builtin_amdgcn_sched_barrier(0);
  // ring slot s & 3 holds stage s ([0] gate, [1] up)
  Iq2Sub W[4][2];
  iq2_sub_load<true>(grow, 0, q, W[0][0]);
  iq2_sub_load<true>(urow, 0, q, W[0][1]);
  iq2_sub_load<true>(grow, 1, q, W[1][0]);
  iq2_sub_load<true>(urow, 1, q, W[1][1]);
  __builtin_amdgcn_sched_barrier(0);
  build_tables8_f16(gb, gt8, mt8);
  const uint16_t* xrow[kXJ];
#pragma unroll
  for (int j = 0; j < kXJ; j++)
    xrow[j] = a.x16 + (size_t)xtok[j] * a.H + 8 * ((tid + kGW * 64 * j) & 15);
  auto x_load = [&](int s) {
    XV r;
#pragma unroll
    for (int j = 0; j < kXJ; j++) r.v[j] = *(const u32x4_t*)(xrow[j] + kGStage * s);
    return r;
  };
  u32x4_t* xtv = (u32x4_t*)&xt[0][0];
  auto x_store = [&](int buf, const XV& x) {
#pragma unroll
    for (int j = 0; j < kXJ; j++) {
      const int c = (tid + kGW * 64 * j) & (kXC - 1), m = c >> 4, ch = c & 15;
      xtv[buf * kXC + m * 16 + (ch ^ (m & 15))] = x.v[j];
    }
  };
  XV X0 = x_load(0), X1 = x_load(1);  // x ring: stage s in X0 (s even) or X1
  __builtin_amdgcn_sched_barrier(0);
  iq2_sub_load<false>(grow, 2, q, W[2][0]);
  iq2_sub_load<false>(urow, 2, q, W[2][1]);
  __builtin_amdgcn_sched_barrier(0);
  x_store(0, X0);
  __syncthreads();  // tables and x of stage 0

  f32x4_t accg[MT], accu[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) accg[mt] = accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* gtab = (const uint8_t*)gt8;
  const uint8_t* stab = (const uint8_t*)mt8;
  float dgp = 1.0f, dup = 1.0f;  // d of the current block (gate, up)
  // stage s = s0 + R (s0 % 4 == 0): block s >> 1 is even for R = 0, 1
  auto stage = [&](int s, auto Rc) {
    constexpr int R = decltype(Rc)::value;
    constexpr bool EVEN = R < 2;
    // requests: x of stage s + 2, weights of stage s + 3 (past the end: a
    // repeat of stage s - 1, which has the same block parity; never used)
    // (x first: a wait for it then never waits for these weights)
    if constexpr ((R & 1) == 0) X0 = x_load(min(s + 2, nst - 1));
    else X1 = x_load(min(s + 2, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    const int sw = s + 3 < nst ? s + 3 : s - 1;
    constexpr bool EVEN3 = ((R + 3) >> 1 & 1) == 0;
    iq2_sub_load<EVEN3>(grow, sw, q, W[(R + 3) & 3][0]);
    iq2_sub_load<EVEN3>(urow, sw, q, W[(R + 3) & 3][1]);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t ig, sg, iu, su;
    float dg, du;
    const uint32_t cg = iq2_sub_words<EVEN>(W[R][0], ig, sg, dg);
    const uint32_t cu = iq2_sub_words<EVEN>(W[R][1], iu, su, du);
    if constexpr ((R & 1) == 0) {  // a block starts: sums in units of its d
      // (hardware reciprocal: within 1 ulp, one rounding per block either way)
      const float rg = dgp * __builtin_amdgcn_rcpf(dg), ru = dup * __builtin_amdgcn_rcpf(du);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        accg[mt] *= rg;
        accu[mt] *= ru;
      }
      dgp = dg;
      dup = du;
    }
    const uint4* xb = xt[R & 1];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f16x8_t fg = iq2_sub_frag(ig, sg, j, cg, rep16, gtab, stab);
      const f16x8_t fu = iq2_sub_frag(iu, su, j, cu, rep16, gtab, stab);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        if (MT > 1 && mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const f16x8_t af = __builtin_bit_cast(f16x8_t, xb[m * 16 + ((4 * q + j) ^ (m & 15))]);
        accg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fg, accg[mt], 0, 0, 0);
        accu[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fu, accu[mt], 0, 0, 0);
      }
    }
    // x of stage s + 1 into the other buffer (after the last stage: unused)
    if constexpr ((R & 1) == 0) x_store(1, X1);
    else x_store(0, X0);
    __syncthreads();
  };
  for (int s0 = 0; s0 < nst; s0 += 4) {
    stage(s0, std::integral_constant<int, 0>{});
    stage(s0 + 1, std::integral_constant<int, 1>{});
    stage(s0 + 2, std::integral_constant<int, 2>{});
    stage(s0 + 3, std::integral_constant<int, 3>{});
  }
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    accg[mt] *= dgp * 0.125f;
    accu[mt] *= dup * 0.125f;
  }
  // the rows' x exponents, loaded only now: held through the main loop they
  // would take the registers of a second block per CU
  uint32_t xe[MT];
  load_row_xexp<MT>(a, row0, q, xe);
  swiglu_store<MT>(a, row0, nrows, mtiles, n, q, accg, accu, n0, kGNF, xe, (uint32_t*)xt[0]);
}

// Small items (at most 16 rows, listed first): as k_grouped_gateup_iq2 with
// MT = 1, but the x tiles sit in an LDS ring of eight stages and the block
// synchronises once per four stages instead of once per stage, so that its
// waves drift apart within a round and their memory, VALU and MFMA phases
// overlap.  During round r (stages 4r .. 4r+3) the ring holds round r's tiles
// (read) and receives round r + 1's: stage s requests x of stage s + 5 and
// stores x of stage s + 4 (requested one stage earlier) into the slot of
// stage s - 4, which every wave finished before the last barrier.
__device__ __attribute__((always_inline)) inline void gateup_iq2_small_body(const GroupArgs& a,
                                                                           int item, uint4* lds) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  uint4* gt8 = lds;                                                   // 32 KB
  uint4* mt8 = lds + 256 * 8;                                         // 16 KB
  u32x4_t (*xr)[16 * 16] = (u32x4_t (*)[16 * 16])(lds + 256 * 8 + 128 * 8);  // 32 KB
  if (item >= a.n_items[1]) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  if (e >= a.E) return;
  const int n0 = blockIdx.x * kGNF;
  if (n0 >= a.I) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  uint32_t xe[1];  // the rows' x exponents, for the epilogue (requested first)
  load_row_xexp<1>(a, row0, q, xe);
  const int n = n0 + 16 * w + (lane & 15);
  const uint32_t rep16 = (uint32_t)(lane & 7) << 4;
  const int rowbytes = (a.H / 256) * kIq2Bytes;
  const uint8_t* grow = a.gate + ((size_t)e * a.I + n) * rowbytes;
  const uint8_t* urow = a.up + ((size_t)e * a.I + n) * rowbytes;
  const int nst = a.H / kGStage;  // a multiple of 4
  // x chunk c = tid & 255 (the upper half of the block repeats the lower):
  // row c >> 4 (past the item: row 0, computed and dropped), column chunk c & 15
  const int c = tid & 255, xm = c >> 4, xch = c & 15;
  const int xslot = xm * 16 + (xch ^ xm);
  // in-order returns: grid bytes and the token, weights of stages 0 and 1,
  // x of stages 0-4, weights of stage 2
  const uint2 gb = *(const uint2*)(a.grid + 8 * (tid & 255));
  const int xtok = a.perm[row0 + (xm < nrows ? xm : 0)] / a.K;
  __builtin_amdgcn_sched_barrier(0);
  Iq2Sub W[4][2];
  iq2_sub_load<true>(grow, 0, q, W[0][0]);
  iq2_sub_load<true>(urow, 0, q, W[0][1]);
  iq2_sub_load<true>(grow, 1, q, W[1][0]);
  iq2_sub_load<true>(urow, 1, q, W[1][1]);
  __builtin_amdgcn_sched_barrier(0);
  build_tables8_f16(gb, gt8, mt8);
  const u32x4_t* xp = (const u32x4_t*)(a.x16 + (size_t)xtok * a.H) + xch;
  auto x_load = [&](int s) { return xp[16 * s]; };
  u32x4_t x0 = x_load(0), x1 = x_load(1), x2 = x_load(2), x3 = x_load(3);
  u32x4_t XA = x_load(min(4, nst - 1)), XB;  // x of stage s + 4 (to store), of s + 5 (in flight)
  __builtin_amdgcn_sched_barrier(0);
  iq2_sub_load<false>(grow, 2, q, W[2][0]);
  iq2_sub_load<false>(urow, 2, q, W[2][1]);
  __builtin_amdgcn_sched_barrier(0);
  xr[0][xslot] = x0;
  xr[1][xslot] = x1;
  xr[2][xslot] = x2;
  xr[3][xslot] = x3;
  __syncthreads();  // tables, x of round 0

  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* gtab = (const uint8_t*)gt8;
  const uint8_t* stab = (const uint8_t*)mt8;
  float dgp = 1.0f, dup = 1.0f;
  const int m = lane & 15;
  auto stage = [&](int s, auto Rc) {
    constexpr int R = decltype(Rc)::value;
    constexpr bool EVEN = R < 2;
    u32x4_t& xin = (R & 1) ? XA : XB;   // receives x of stage s + 5
    u32x4_t& xout = (R & 1) ? XB : XA;  // holds x of stage s + 4
    xin = x_load(min(s + 5, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    const int sw = s + 3 < nst ? s + 3 : s - 1;
    constexpr bool EVEN3 = ((R + 3) >> 1 & 1) == 0;
    iq2_sub_load<EVEN3>(grow, sw, q, W[(R + 3) & 3][0]);
    iq2_sub_load<EVEN3>(urow, sw, q, W[(R + 3) & 3][1]);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t ig, sg, iu, su;
    float dg, du;
    const uint32_t cg = iq2_sub_words<EVEN>(W[R][0], ig, sg, dg);
    const uint32_t cu = iq2_sub_words<EVEN>(W[R][1], iu, su, du);
    if constexpr ((R & 1) == 0) {  // a block starts: sums in units of its d
      // (hardware reciprocal: within 1 ulp, one rounding per block either way)
      const float rg = dgp * __builtin_amdgcn_rcpf(dg), ru = dup * __builtin_amdgcn_rcpf(du);
      accg *= rg;
      accu *= ru;
      dgp = dg;
      dup = du;
    }
    const u32x4_t* xb = xr[s & 7];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const f16x8_t fg = iq2_sub_frag(ig, sg, j, cg, rep16, gtab, stab);
      const f16x8_t fu = iq2_sub_frag(iu, su, j, cu, rep16, gtab, stab);
      const f16x8_t af = __builtin_bit_cast(f16x8_t, xb[m * 16 + ((4 * q + j) ^ m)]);
      accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fg, accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fu, accu, 0, 0, 0);
    }
    xr[(s + 4) & 7][xslot] = xout;  // past the last stage: unused
    if constexpr (R == 3) __syncthreads();
  };
  for (int s0 = 0; s0 < nst; s0 += 4) {
    stage(s0, std::integral_constant<int, 0>{});
    stage(s0 + 1, std::integral_constant<int, 1>{});
    stage(s0 + 2, std::integral_constant<int, 2>{});
    stage(s0 + 3, std::integral_constant<int, 3>{});
  }
  f32x4_t ag[1] = {accg * (dgp * 0.125f)}, au[1] = {accu * (dup * 0.125f)};
  swiglu_store<1>(a, row0, nrows, 1, n, q, ag, au, n0, kGNF, xe, (uint32_t*)xr[0]);
}

__global__ __launch_bounds__(kGW * 64) void k_grouped_gateup_iq2_small(GroupArgs a) {
  __shared__ uint4 lds[kGuLds];
  gateup_iq2_small_body(a, (int)blockIdx.y, lds);
}

// Every routed IQ2_XXS gate/up item in one launch: grid rows first take the
// items after the small ones (64-row pieces, the longest blocks, started
// first), then the small items, so that the two kinds share the chip instead
// of the 64-row items running alone after the small ones.  Four waves per
// SIMD (two blocks per CU, as each body alone) bound the registers.
__global__ __launch_bounds__(kGW * 64, 4) void k_grouped_gateup_iq2_all(GroupArgs a) {
  __shared__ uint4 lds[kGuLds];
  const int n_small = a.n_items[1], n_rest = a.n_items[0] - n_small;
  const int y = (int)blockIdx.y;
  if (y < n_rest) gateup_iq2_body<4>(a, n_small + y, lds);
  else gateup_iq2_small_body(a, y - n_rest, lds);
}

// x (bf16) -> binary16 for the grouped IQ2_XXS and Q4_K gate/up kernels,
// one block per token: the token's values are scaled by the power of two
// 2^e that brings their largest magnitude into [2^13, 2^14), exact for bf16
// values (8 significant bits) down to 2^-14 of binary16's normal range; e
// goes to byte r of word j - r of xrexp for each of the token's K sorted
// rows j = inv[t*K + k] (r = 0..3, j - r >= 0).  NaN or
// infinite values propagate (e = 0).  hidden is a multiple of 8; up to 8192
// columns a thread's chunks stay in registers between the two passes.
constexpr int kXRegChunks = 4;
__global__ __launch_bounds__(256) void k_x_to_f16(const uint16_t* __restrict__ x, int H, int K,
                                                 const int32_t* __restrict__ inv,
                                                 uint16_t* __restrict__ x16,
                                                 int8_t* __restrict__ xrexp) {
  __shared__ uint32_t s_max[2][4];
  const int t = blockIdx.x, tid = threadIdx.x, n8 = H / 8;
  const uint4* xt = (const uint4*)(x + (size_t)t * H);
  const bool regs = n8 <= 256 * kXRegChunks;
  uint4 xv[kXRegChunks];
  AbsMax am;
  auto take = [&](uint4 v) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      am.add(__uint_as_float(in[k] << 16));
      am.add(__uint_as_float(in[k] & 0xFFFF0000u));
    }
  };
  if (regs) {
#pragma unroll
    for (int j = 0; j < kXRegChunks; j++) {
      const int i = tid + 256 * j;
      xv[j] = i < n8 ? xt[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kXRegChunks; j++) take(xv[j]);
  } else {
    for (int i = tid; i < n8; i += 256) take(xt[i]);
  }
  am = wave_absmax(am);
  if ((tid & 63) == 0) {
    s_max[0][tid >> 6] = (uint32_t)am.smax;
    s_max[1][tid >> 6] = am.umax;
  }
  __syncthreads();
  AbsMax bm;
  for (int i = 0; i < 4; i++) {
    bm.smax = max(bm.smax, (int)s_max[0][i]);
    bm.umax = max(bm.umax, s_max[1][i]);
  }
  bool bad;
  const float M = bm.value(bad);
  const int e = pow2_exponent(M, bad, 13);
  for (int i = tid; i < 4 * K; i += 256) {
    const int j = inv[t * K + (i >> 2)], r = i & 3;
    if (j >= r) xrexp[4 * (size_t)(j - r) + r] = (int8_t)e;
  }
  auto put = [&](int i, uint4 v) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const float lo = ldexpf(__uint_as_float(in[k] << 16), e);
      const float hi = ldexpf(__uint_as_float(in[k] & 0xFFFF0000u), e);
      o[k] = f32_to_f16_bits(lo) | (f32_to_f16_bits(hi) << 16);
    }
    ((uint4*)(x16 + (size_t)t * H))[i] = make_uint4(o[0], o[1], o[2], o[3]);
  };
  if (regs) {
#pragma unroll
    for (int j = 0; j < kXRegChunks; j++)
      if (tid + 256 * j < n8) put(tid + 256 * j, xv[j]);
  } else {
    for (int i = tid; i < n8; i += 256) put(i, xt[i]);  // the second read hits the cache
  }
}

// ---------------------------------------------------------------------------
// gate/up of the shared expert (Q8_0 gate and up), software-pipelined like
// k_grouped_gateup_iq2.  Stages of 64 columns (two Q8_0 blocks); per block a
// lane holds the three aligned words covering its 8 codes and the word with
// d.  B = the codes in bf16 (exact), the block scale multiplies each result.
struct Q80Stage {
  uint32_t c[2][3];
  uint32_t dw[2];
};

__device__ inline void q80_stage_load(const uint8_t* __restrict__ row, int s, int q, Q80Stage& st) {
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int b = 2 * s + i;
    const int start = kQ80Bytes * b + 2 + 8 * q;
    const int sh = start & 3;
    const uint32_t* p = (const uint32_t*)(row + (start - sh));
    st.c[i][0] = p[0];
    st.c[i][1] = p[1];
    st.c[i][2] = p[sh ? 2 : 1];  // never past the row when not needed
    st.dw[i] = *(const uint32_t*)(row + ((kQ80Bytes * b) & ~3));
  }
}

// block i (0, 1) of a stage: (2i + 2) & 3 is the codes' misalignment, (2i) & 3
// the position of d
__device__ inline bf16x8_t q80_stage_frag(const Q80Stage& st, int i, float& scale) {
  const uint32_t sh = i ? 0u : 2u;
  const uint32_t c0 = align_bytes(st.c[i][1], st.c[i][0], sh);
  const uint32_t c1 = align_bytes(st.c[i][2], st.c[i][1], sh);
  scale = f16_bits_to_f32(i ? (st.dw[i] >> 16) : (st.dw[i] & 0xFFFFu));
  uint4 v;
  i8x4_to_bf16x4(c0, v.x, v.y);
  i8x4_to_bf16x4(c1, v.z, v.w);
  return __builtin_bit_cast(bf16x8_t, v);
}

__global__ __launch_bounds__(kGW * 64) void k_grouped_gateup_q80(GroupArgs a) {
  __shared__ uint4 xt[2][kMC * 8];  // 2 x 8 KB: row m, 16-byte chunk c at m*8 + (c ^ ((m >> 1) & 7))
  __shared__ int tok[kMC];
  const int item = grid_item(a);
  if (item >= *a.n_items) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  if (e != a.E) return;  // the shared expert only
  const int n0 = blockIdx.x * kGNF;
  if (n0 >= a.sh_I) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  const int n = n0 + 16 * w + (lane & 15);
  const int rowbytes = (a.H / 32) * kQ80Bytes;
  const uint8_t* grow = a.sh_gate + (size_t)n * rowbytes;
  const uint8_t* urow = a.sh_up + (size_t)n * rowbytes;
  // this block's share of the K stages (a.ksplit_g blocks along z)
  const int nall = a.H / 64, nsp = nall / a.ksplit_g, s0 = blockIdx.z * nsp;
  const int mtiles = (nrows + 15) >> 4;
  Q80Stage cg, cu;
  q80_stage_load(grow, s0, q, cg);
  q80_stage_load(urow, s0, q, cu);
  if (tid < kMC) tok[tid] = tid < nrows ? row_token(a, row0 + tid) : -1;
  __syncthreads();
  // x tile of a stage: thread -> row tid >> 3, chunk tid & 7
  const int xm = tid >> 3, xc = tid & 7;
  auto x_load = [&](int s) -> uint4 {
    return xm < nrows ? ((const uint4*)(a.x + (size_t)tok[xm] * a.H + 64 * s))[xc]
                      : make_uint4(0, 0, 0, 0);
  };
  auto x_store = [&](int buf, uint4 v) { xt[buf][xm * 8 + (xc ^ ((xm >> 1) & 7))] = v; };
  x_store(s0 & 1, x_load(s0));
  __syncthreads();
  f32x4_t accg[4], accu[4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) accg[mt] = accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s0 + nsp; s++) {
    const bool more = s + 1 < s0 + nsp;
    Q80Stage ng, nu;
    uint4 xv = make_uint4(0, 0, 0, 0);
    if (more) {
      q80_stage_load(grow, s + 1, q, ng);
      q80_stage_load(urow, s + 1, q, nu);
      xv = x_load(s + 1);
    }
    const uint4* xb = xt[s & 1];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      float sg, su;
      const bf16x8_t fg = q80_stage_frag(cg, i, sg);
      const bf16x8_t fu = q80_stage_frag(cu, i, su);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        if (mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const bf16x8_t af =
            __builtin_bit_cast(bf16x8_t, xb[m * 8 + ((4 * i + q) ^ ((m >> 1) & 7))]);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, fg, z, 0, 0, 0);
        const f32x4_t tu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, fu, z, 0, 0, 0);
        accg[mt] += sg * tg;
        accu[mt] += su * tu;
      }
    }
    if (more) {
      x_store((s + 1) & 1, xv);
      cg = ng;
      cu = nu;
    }
    __syncthreads();
  }
  if (a.ksplit_g == 1) {
    swiglu_store(a, row0, nrows, mtiles, n, q, accg, accu, n0, kGNF, nullptr, (uint32_t*)xt[0]);
    return;
  }
  // partial sums of this K share: part[z][row - T*K][f] (gate), [.. + I] (up)
  const int TK = a.T * a.K;
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (mt >= mtiles) break;
      const int m = 16 * mt + 4 * q + r;
      if (m < nrows) {
        float* pp = a.part + ((size_t)blockIdx.z * a.T + (row0 + m - TK)) * 2 * a.sh_I;
        pp[n] = accg[mt][r];
        pp[a.sh_I + n] = accu[mt][r];
      }
    }
}

// Reduces the K shares of the shared expert's gate/up in a fixed order and
// writes the SwiGLU rows like swiglu_store: binary16 high/low parts and the
// sums of 16 consecutive features (DPP inside each row of 16 lanes).  One
// thread per (token, feature); all loads of a thread are issued together.
constexpr int kMaxSplit = 16;
__global__ __launch_bounds__(256) void k_swiglu_finish(GroupArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int I = a.sh_I;
  const bool live = idx < a.T * I;
  const int t = live ? idx / I : 0, f = live ? idx % I : 0;
  float gp[kMaxSplit], up[kMaxSplit];
#pragma unroll
  for (int z = 0; z < kMaxSplit; z++) {
    const float* pp = a.part + ((size_t)z * a.T + t) * 2 * I;
    const bool use = live && z < a.ksplit_g;
    gp[z] = use ? pp[f] : 0.0f;
    up[z] = use ? pp[I + f] : 0.0f;
  }
  float g = 0.0f, u = 0.0f;
#pragma unroll
  for (int z = 0; z < kMaxSplit; z++) {
    g += gp[z];
    u += up[z];
  }
  const float v0 = live ? silu(g) * u : 0.0f;
  // one exponent per 64-feature range of the row (a wave: I is a multiple of
  // 64, so no range straddles two rows), chosen as in swiglu_store
  AbsMax am;
  if (live) am.add(v0);
  am = wave_absmax(am);
  bool bad;
  const float M = am.value(bad);
  const int e = M < 2048.0f ? 0 : pow2_exponent(M, bad, 10);
  const float v = ldexpf(v0, e);
  float sum = v;
  sum += dpp_f32<0xB1>(sum);
  sum += dpp_f32<0x4E>(sum);
  sum += dpp_f32<0x141>(sum);
  sum += dpp_f32<0x140>(sum);
  if (!live) return;
  const size_t row = (size_t)a.T * a.K + t;
  const uint32_t hi = f32_to_f16_bits(v);
  a.hh[row * a.I + f] = (uint16_t)hi;
  a.hl[row * a.I + f] = (uint16_t)f32_to_f16_bits(v - f16_bits_to_f32(hi));
  if ((f & 15) == 0) {
    const uint32_t shi = f32_to_f16_bits(sum);
    a.hsh[row * (a.I / 16) + f / 16] = (uint16_t)shi;
    a.hsl[row * (a.I / 16) + f / 16] = (uint16_t)f32_to_f16_bits(sum - f16_bits_to_f32(shi));
  }
  if ((f & 63) == 0) a.hexp[row * (a.I / 64) + f / 64] = (int8_t)e;
}

// down for one work item and 64 output features.  Grid (H/64, max_items).
// A (the SwiGLU rows) is staged per 256 columns as f16 hi/lo tiles with the
// same swizzle as above, plus per-16-column sums (hi/lo) for the min term.
__global__ __launch_bounds__(256) void k_grouped_down(GroupArgs a) {
  __shared__ uint4 ah[kMC * 32];
  __shared__ uint4 al[kMC * 32];
  __shared__ uint2 sh_hi[kMC * 4];  // [m][4 x (4 f16)] sub-block sums, hi part
  __shared__ uint2 sh_lo[kMC * 4];
  __shared__ int s_eb[kMC];         // row m's binary16 exponent in the staged block
  const int item = grid_item(a);
  if (item >= *a.n_items) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  const bool shr = e == a.E;
  // routed Q2_K and Q4_K items run in k_grouped_down_q2k / _q4k; only the
  // shared expert is split along K (grid z)
  if (!shr && (q2k_grouped_fast(a) || q4k_grouped_dn(a) || blockIdx.z > 0)) return;
  const int I = shr ? a.sh_I : a.I;
  const int qd = shr ? a.sh_qt_d : a.qt_d;
  const uint8_t* D = shr ? a.sh_down : a.down;
  const int ee = shr ? 0 : e;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  const int n = blockIdx.x * kNT + 16 * w + (lane & 15);
  const int nb = I / 256;
  const int bbd = block_bytes(qd) * (256 / block_values(qd));
  const int mtiles = (nrows + 15) >> 4;
  f32x4_t acc[4];
  for (int mt = 0; mt < 4; mt++) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the accumulators of row 16 mt + 4 q + r are in units of 2^eb[mt][r], the
  // exponent of that row's current block
  int eb[4][4] = {};
  const size_t rowd = (size_t)ee * a.H + n;
  // K share (shared-expert split, a.ksplit_d blocks along z)
  const int ks = shr ? a.ksplit_d : 1, nbs = nb / ks, kb0 = blockIdx.z * nbs;
  for (int kb = kb0; kb < kb0 + nbs; kb++) {
    // Q4_K: the block's header and the lane's code bytes are requested before
    // the h tile is staged, so that the two loads overlap
    uint4 q4h = make_uint4(0, 0, 0, 0);
    uint2 q4c[4] = {};
    if (qd == DS4MOE_Q4_K) {
      const uint8_t* qb = D + (rowd * nb + kb) * bbd;
      q4h = *(const uint4*)qb;
#pragma unroll
      for (int c = 0; c < 4; c++) q4c[c] = *(const uint2*)(qb + 16 + 32 * c + 8 * q);
    }
    // stage: thread -> (row m, 16-column sub-block j): 16 values, high and low
    // parts, brought to the block's largest exponent (the smallest e of its
    // four 64-feature ranges) when its range has another one
    for (int c = tid; c < kMC * 16; c += 256) {
      const int m = c >> 4, j = c & 15;
      uint4 h0 = make_uint4(0, 0, 0, 0), h1 = h0, l0 = h0, l1 = h0;
      uint16_t sh16 = 0, sl16 = 0;
      if (m < nrows) {
        const size_t row = (size_t)(row0 + m);
        const uint4* hp = (const uint4*)(a.hh + row * a.I + 256 * kb + 16 * j);
        const uint4* lp = (const uint4*)(a.hl + row * a.I + 256 * kb + 16 * j);
        h0 = hp[0];
        h1 = hp[1];
        l0 = lp[0];
        l1 = lp[1];
        sh16 = a.hsh[row * (a.I / 16) + 16 * kb + j];
        sl16 = a.hsl[row * (a.I / 16) + 16 * kb + j];
        const uint32_t ew = *(const uint32_t*)(a.hexp + row * (a.I / 64) + 4 * kb);
        const int e0 = (int8_t)(ew & 0xFF), e1 = (int8_t)((ew >> 8) & 0xFF),
                  e2 = (int8_t)((ew >> 16) & 0xFF), e3 = (int8_t)(ew >> 24);
        const int emin = min(min(e0, e1), min(e2, e3));
        const int er = (int8_t)((ew >> (8 * (j >> 2))) & 0xFF);
        if (er != emin) {  // rescale the pair (hi, lo) exactly, then split again
          const int de = emin - er;
          auto fix = [&](uint32_t& hw, uint32_t& lw) {
            const float v0 = ldexpf(f16_bits_to_f32(hw & 0xFFFFu) + f16_bits_to_f32(lw & 0xFFFFu), de);
            const float v1 = ldexpf(f16_bits_to_f32(hw >> 16) + f16_bits_to_f32(lw >> 16), de);
            const uint32_t a0 = f32_to_f16_bits(v0), a1 = f32_to_f16_bits(v1);
            hw = a0 | (a1 << 16);
            lw = f32_to_f16_bits(v0 - f16_bits_to_f32(a0)) | (f32_to_f16_bits(v1 - f16_bits_to_f32(a1)) << 16);
          };
          fix(h0.x, l0.x);
          fix(h0.y, l0.y);
          fix(h0.z, l0.z);
          fix(h0.w, l0.w);
          fix(h1.x, l1.x);
          fix(h1.y, l1.y);
          fix(h1.z, l1.z);
          fix(h1.w, l1.w);
          const float sv = ldexpf(f16_bits_to_f32(sh16) + f16_bits_to_f32(sl16), de);
          sh16 = (uint16_t)f32_to_f16_bits(sv);
          sl16 = (uint16_t)f32_to_f16_bits(sv - f16_bits_to_f32(sh16));
        }
        if (j == 0) s_eb[m] = emin;
      }
      // two 16-byte chunks (8 values each) per sub-block
      const int c0 = 2 * j, c1 = 2 * j + 1;
      ah[m * 32 + (c0 ^ (m & 15))] = h0;
      ah[m * 32 + (c1 ^ (m & 15))] = h1;
      al[m * 32 + (c0 ^ (m & 15))] = l0;
      al[m * 32 + (c1 ^ (m & 15))] = l1;
      ((uint16_t*)sh_hi)[m * 16 + j] = sh16;
      ((uint16_t*)sh_lo)[m * 16 + j] = sl16;
    }
    __syncthreads();
    // the accumulators follow their rows' exponents (exact rescaling)
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = 16 * mt + 4 * q + r;
        const int en = m < nrows ? s_eb[m] : 0;
        acc[mt][r] = ldexpf(acc[mt][r], en - eb[mt][r]);
        eb[mt][r] = en;
      }
    const uint8_t* blk = D + (rowd * nb + kb) * bbd;
    if (qd == DS4MOE_Q2_K) {
      // lane: output row n, k = 4q + j inside each 16-value sub-block
      uint32_t qs4[4];  // qs dwords at 32hh + 16p + 4q, index 2hh + p
      for (int hh = 0; hh < 2; hh++)
        for (int p = 0; p < 2; p++) qs4[2 * hh + p] = *(const uint32_t*)(blk + 16 + 32 * hh + 16 * p + 4 * q);
      const uint4 scv = *(const uint4*)blk;
      const uint32_t scw[4] = {scv.x, scv.y, scv.z, scv.w};
      const uint32_t dd = *(const uint32_t*)(blk + 80);
      const float d = f16_bits_to_f32(dd & 0xFFFFu), dmin = f16_bits_to_f32(dd >> 16);
      uint32_t pk[8];  // 16-bit lanes holding whole code bytes: (j0,j1), (j2,j3)
      for (int i = 0; i < 4; i++) {
        pk[2 * i] = vperm(0u, qs4[i], 0x0C010C00u);
        pk[2 * i + 1] = vperm(0u, qs4[i], 0x0C030C02u);
      }
#pragma unroll 1
      for (int sb = 0; sb < 16; sb++) {
        const int hh = sb >> 3, s = (sb >> 1) & 3, p = sb & 1;
        const uint32_t mk = 0x00030003u << (2 * s);
        const int ix = 2 * (2 * hh + p);
        const uint32_t b0 = pk[ix] & mk, b1 = pk[ix + 1] & mk;
        const f16x4_t bf = __builtin_bit_cast(f16x4_t, make_uint2(b0, b1));
        const uint32_t scb = (scw[sb >> 2] >> (8 * (sb & 3))) & 0xFu;
        const float mult = d * (float)scb * (16777216.0f / (float)(1 << (2 * s)));
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          if (mt >= mtiles) break;
          const int m = 16 * mt + (lane & 15);
          // A fragment: 4 values k = 4q..4q+3 of sub-block sb = half of 16-byte chunk 2sb + q/2
          const uint4 ch = ah[m * 32 + ((2 * sb + (q >> 1)) ^ (m & 15))];
          const uint4 cl = al[m * 32 + ((2 * sb + (q >> 1)) ^ (m & 15))];
          const uint2 fh = (q & 1) ? make_uint2(ch.z, ch.w) : make_uint2(ch.x, ch.y);
          const uint2 fl = (q & 1) ? make_uint2(cl.z, cl.w) : make_uint2(cl.x, cl.y);
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, fh), bf, z, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, fl), bf, t, 0, 0, 0);
          acc[mt] += mult * t;
        }
      }
      // mins: sum_j m_j * hsum_j over the block's 16 sub-blocks, k = sub-block
      const uint32_t scq = scw[q];
      const uint32_t mn = (scq >> 4) & 0x0F0F0F0Fu;  // min nibbles of sub-blocks 4q..4q+3
      const uint32_t m0 = vperm(0u, mn, 0x0C010C00u), m1 = vperm(0u, mn, 0x0C030C02u);
      const f16x4_t bm = __builtin_bit_cast(f16x4_t, make_uint2(m0, m1));
      const float mmult = dmin * 16777216.0f;
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        if (mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, sh_hi[m * 4 + q]), bm, z, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, sh_lo[m * 4 + q]), bm, t, 0, 0, 0);
        acc[mt] -= mmult * t;
      }
    } else if (qd == DS4MOE_Q4_K) {
      // Q4_K: group j = 2c (low nibbles) and 2c + 1 (high) of code chunk c
      const uint4 hd = q4h;
      const float d = f16_bits_to_f32(hd.x & 0xFFFFu), dmin = f16_bits_to_f32(hd.x >> 16);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const uint4 pc = q4k_pairs(q4c[c]);
#pragma unroll
        for (int hi = 0; hi < 2; hi++) {
          const int j = 2 * c + hi;
          int sc, mn;
          q4k_scale_min(hd, j, sc, mn);
          const float mult = d * (float)sc * (hi ? 1048576.0f : 16777216.0f);
          const f16x8_t bf = q4k_frag(pc, hi);
#pragma unroll
          for (int mt = 0; mt < 4; mt++) {
            if (mt >= mtiles) break;
            const int m = 16 * mt + (lane & 15);
            const f16x8_t fh = __builtin_bit_cast(f16x8_t, ah[m * 32 + ((4 * j + q) ^ (m & 15))]);
            const f16x8_t fl = __builtin_bit_cast(f16x8_t, al[m * 32 + ((4 * j + q) ^ (m & 15))]);
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(fh, bf, z, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(fl, bf, t, 0, 0, 0);
            acc[mt] += mult * t;
          }
        }
      }
      // mins: the 16-feature sums j' = 4q .. 4q+3 belong to groups 2q, 2q+1
      int sc0, m0, m1;
      q4k_scale_min(hd, 2 * q, sc0, m0);
      q4k_scale_min(hd, 2 * q + 1, sc0, m1);
      const uint32_t f0 = f32_to_f16_bits((float)m0), f1 = f32_to_f16_bits((float)m1);
      const f16x4_t bm = __builtin_bit_cast(f16x4_t, make_uint2(f0 | (f0 << 16), f1 | (f1 << 16)));
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        if (mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, sh_hi[m * 4 + q]), bm, z, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, sh_lo[m * 4 + q]), bm, t, 0, 0, 0);
        acc[mt] -= dmin * t;
      }
    } else {
      // Q8_0 (shared expert): 32-value blocks, f16 MFMA 16x16x32
#pragma unroll 1
      for (int g = 0; g < 8; g++) {
        const uint8_t* bp = blk + g * kQ80Bytes;
        const float dq = f16_bits_to_f32((uint32_t)((const uint16_t*)bp)[0]);
        const uint2 c = load8_a2(bp + 2 + 8 * q);
        uint4 v;
        i8x4_to_f16x4(c.x, v.x, v.y);
        i8x4_to_f16x4(c.y, v.z, v.w);
        const f16x8_t bf = __builtin_bit_cast(f16x8_t, v);
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          if (mt >= mtiles) break;
          const int m = 16 * mt + (lane & 15);
          const f16x8_t fh = __builtin_bit_cast(f16x8_t, ah[m * 32 + ((4 * g + q) ^ (m & 15))]);
          const f16x8_t fl = __builtin_bit_cast(f16x8_t, al[m * 32 + ((4 * g + q) ^ (m & 15))]);
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(fh, bf, z, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_f16(fl, bf, t, 0, 0, 0);
          acc[mt] += dq * t;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (mt >= mtiles) break;
      const int m = 16 * mt + 4 * q + r;
      if (m < nrows) {
        const float y = ldexpf(acc[mt][r], -eb[mt][r]);
        if (ks == 1) a.y[(size_t)(row0 + m) * a.H + n] = y;
        else a.part[((size_t)blockIdx.z * a.T + (row0 + m - a.T * a.K)) * a.H + n] = y;
      }
    }
}

// down for routed items with Q2_K down weights: software-pipelined.
// Grid (H/128, items), 512 threads; wave w owns output features
// n0 + 16w .. +15.  K runs in stages of 128 columns (half a Q2_K block: its
// 32 code bytes hold four 2-bit planes of 32 columns each).  In a stage,
// lane quarter q takes code bytes 8q .. 8q+7 of the half: plane j of them is
// the B fragment of MFMA step j (f16 16x16x32), columns 32j + 8q .. +7 of
// the stage, all in one 16-value sub-block, so its scale nibble goes into B:
//   B = q * sc as a binary16 subnormal (q * sc * 2^-24, exact),
//   A = the SwiGLU rows as binary16 high and low parts (two MFMAs),
// and, as in the IQ2_XXS gate/up kernel, the accumulators hold the sum in
// units of the current block's d (rescaled at each block start).  The mins:
// per stage one f16 16x16x16 MFMA of the eight sub-block sums of h (hi, lo;
// written by gate/up) against the min nibbles (quarters 0 and 1; B = 0 in
// quarters 2 and 3), scaled by dmin / d.  Weights of stage s + 3 and the h
// tile (with the sums) of stage s + 2 are in flight while stage s is
// multiplied; one barrier per stage.
struct Q2kSub {
  uint32_t c0, c1, s0, s1, dd;  // the lane's code bytes, the half's scale bytes, d | dmin << 16
};

__device__ inline void q2k_sub_load(const uint8_t* __restrict__ row, int s, int q, Q2kSub& o) {
  const uint8_t* blk = row + kQ2kBytes * (s >> 1);
  const int hf = s & 1;
  const uint32_t* c = (const uint32_t*)(blk + 16 + 32 * hf + 8 * q);
  o.c0 = c[0];
  o.c1 = c[1];
  const uint32_t* sc = (const uint32_t*)(blk + 8 * hf);
  o.s0 = sc[0];
  o.s1 = sc[1];
  o.dd = *(const uint32_t*)(blk + 80);
}

// MT = 1: the small items (at most 16 rows, listed first); MT = 4: the rest.
template <int MT>
__global__ __launch_bounds__(kDW * 64) void k_grouped_down_q2k(GroupArgs a) {
  constexpr int kRows = 16 * MT;
  constexpr int kHC = kRows * 32;                          // h chunks of a stage (hi, lo)
  constexpr int kHJ = (kHC + kDW * 64 - 1) / (kDW * 64);  // per thread
  constexpr int kSC = kRows * 2;                           // sum chunks (hi, lo)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ u32x4_t ht[2][kHC];  // row m: [hi 16 chunks][lo 16 chunks], chunk c at c ^ (m & 15)
  __shared__ u32x4_t st[2][kSC];  // row m: [8 sums hi][8 sums lo]
  const int n_small = a.n_items[1];
  const int item = (MT == 1 ? 0 : n_small) + (int)blockIdx.y;
  if (item >= (MT == 1 ? n_small : a.n_items[0])) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  if (e >= a.E) return;  // shared-expert items run in k_grouped_down
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  const int n = blockIdx.x * kDNF + 16 * w + (lane & 15);
  const int rowbytes = (a.I / 256) * kQ2kBytes;
  const uint8_t* drow = a.down + ((size_t)e * a.H + n) * rowbytes;
  const int nst = a.I / 128;  // a multiple of 4
  const int mtiles = (nrows + 15) >> 4;
  // h tile loads: chunk c = tid + 512 j -> row c >> 5, part (c >> 4) & 1,
  // chunk c & 15; sum chunk cs = tid mod 2 kRows -> row cs >> 1, part cs & 1.
  // Rows past the item repeat row 0 (never stored); threads past a tile load
  // and store a chunk again: no branches around loads or stores.
  struct HV {
    u32x4_t v[kHJ];
    u32x4_t sm;
  };
  const uint16_t* hsrc[kHJ];
#pragma unroll
  for (int j = 0; j < kHJ; j++) {
    const int c = (tid + kDW * 64 * j) & (kHC - 1), m = c >> 5;
    const size_t r = (size_t)(row0 + (m < nrows ? m : 0));
    hsrc[j] = ((c >> 4) & 1 ? a.hl : a.hh) + r * a.I + 8 * (c & 15);
  }
  const int cs = tid & (kSC - 1), ms = cs >> 1;
  const uint16_t* ssrc = ((cs & 1) ? a.hsl : a.hsh) + (size_t)(row0 + (ms < nrows ? ms : 0)) * (a.I / 16);
  auto h_load = [&](int s) {
    HV r;
#pragma unroll
    for (int j = 0; j < kHJ; j++) r.v[j] = *(const u32x4_t*)(hsrc[j] + 128 * s);
    r.sm = *(const u32x4_t*)(ssrc + 8 * s);
    return r;
  };
  auto h_store = [&](int buf, const HV& h) {
#pragma unroll
    for (int j = 0; j < kHJ; j++) {
      const int c = (tid + kDW * 64 * j) & (kHC - 1), m = c >> 5;
      ht[buf][m * 32 + (c & 16) + ((c & 15) ^ (m & 15))] = h.v[j];
    }
    st[buf][cs] = h.sm;
  };
  // in-order returns: weights of stages 0 and 1, h of stages 0 and 1, then
  // the weights of stage 2 (in the loop, as in the first stage, h then weights)
  Q2kSub W[4];
  q2k_sub_load(drow, 0, q, W[0]);
  q2k_sub_load(drow, 1, q, W[1]);
  __builtin_amdgcn_sched_barrier(0);
  HV H0 = h_load(0), H1 = h_load(1);
  __builtin_amdgcn_sched_barrier(0);
  q2k_sub_load(drow, 2, q, W[2]);
  __builtin_amdgcn_sched_barrier(0);
  h_store(0, H0);
  __syncthreads();

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float dp = 1.0f;  // d of the current block
  // the stored rows are h * 2^e(stage), e the same for every row of the item
  // (byte 2s of the item's first row): the accumulators hold the sum in
  // units of the current stage's 2^e too.  Read through the scalar cache,
  // four stages ahead, so that no wait for them waits for vector loads.
  const int32_t* ex32 = (const int32_t*)(a.hexp + (size_t)row0 * (a.I / 64));
  int ecur0 = load_scalar_i32(ex32, 0), ecur1 = load_scalar_i32(ex32, 1);
  int ep = (int8_t)(ecur0 & 0xFF);
  auto stage = [&](int s, auto Rc) {
    constexpr int R = decltype(Rc)::value;
    if constexpr ((R & 1) == 0) H0 = h_load(min(s + 2, nst - 1));
    else H1 = h_load(min(s + 2, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    q2k_sub_load(drow, s + 3 < nst ? s + 3 : s - 1, q, W[(R + 3) & 3]);
    __builtin_amdgcn_sched_barrier(0);
    const Q2kSub& cw = W[R];
    const float dv = f16_bits_to_f32(cw.dd & 0xFFFFu);
    const float d = dv != 0.0f ? dv : 1.0f;
    const float rd = __builtin_amdgcn_rcpf(d);  // within 1 ulp
    const int es = (int8_t)(((R < 2 ? ecur0 : ecur1) >> (16 * (R & 1))) & 0xFF), de = es - ep;
    ep = es;
    if constexpr ((R & 1) == 0) {  // a block starts: sums in units of its d
      const float r = ldexpf(dp * rd, de);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[mt] *= r;
      dp = d;
    } else if (de != 0) {
      const float r = ldexpf(1.0f, de);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[mt] *= r;
    }
    // scale bytes 2j + (q >> 1) of the half (sub-block 8hf + 2j + (q >> 1))
    const uint32_t s4 = vperm(cw.s1, cw.s0, (q >> 1) ? 0x07050301u : 0x06040200u);
    const uint32_t scm = dv != 0.0f ? s4 & 0x0F0F0F0Fu : 0u;
    // code bytes in 16-bit lanes: (b0, b1), (b2, b3), (b4, b5), (b6, b7)
    const uint32_t P0 = vperm(0u, cw.c0, 0x0C010C00u), P1 = vperm(0u, cw.c0, 0x0C030C02u);
    const uint32_t P2 = vperm(0u, cw.c1, 0x0C010C00u), P3 = vperm(0u, cw.c1, 0x0C030C02u);
    const u32x4_t* hb = ht[R & 1];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint32_t sc = (scm >> (8 * j)) & 0xFFu;
      // q * sc < 46 in each 16-bit lane: the binary16 subnormal q sc 2^-24
      const uint4 bv = make_uint4(__mul24((P0 >> (2 * j)) & 0x00030003u, sc),
                                  __mul24((P1 >> (2 * j)) & 0x00030003u, sc),
                                  __mul24((P2 >> (2 * j)) & 0x00030003u, sc),
                                  __mul24((P3 >> (2 * j)) & 0x00030003u, sc));
      const f16x8_t bf = __builtin_bit_cast(f16x8_t, bv);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        if (MT > 1 && mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const int c = (4 * j + q) ^ (m & 15);
        const f16x8_t ahi = __builtin_bit_cast(f16x8_t, hb[m * 32 + c]);
        const f16x8_t alo = __builtin_bit_cast(f16x8_t, hb[m * 32 + 16 + c]);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bf, acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bf, acc[mt], 0, 0, 0);
      }
    }
    // mins of the half's eight sub-blocks: quarter q < 2 holds 4q .. 4q+3
    {
      const uint32_t mn = ((q & 1) ? cw.s1 : cw.s0) >> 4 & 0x0F0F0F0Fu;
      const uint32_t m0 = q < 2 ? vperm(0u, mn, 0x0C010C00u) : 0u;
      const uint32_t m1 = q < 2 ? vperm(0u, mn, 0x0C030C02u) : 0u;
      const f16x4_t bm = __builtin_bit_cast(f16x4_t, make_uint2(m0, m1));
      const float fmin = f16_bits_to_f32(cw.dd >> 16) * rd;
      const u32x4_t* sb = st[R & 1];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        if (MT > 1 && mt >= mtiles) break;
        const int m = 16 * mt + (lane & 15);
        const uint2* sp = (const uint2*)&sb[2 * m];
        const uint2 shi = sp[q & 1], slo = sp[2 + (q & 1)];
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, shi), bm, z, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, slo), bm, t, 0, 0, 0);
        acc[mt] -= fmin * t;
      }
    }
    // h of stage s + 1 into the other buffers (after the last stage: unused)
    if constexpr ((R & 1) == 0) h_store(1, H1);
    else h_store(0, H0);
    __syncthreads();
  };
  for (int s0 = 0; s0 < nst; s0 += 4) {
    const int sn = s0 + 4 < nst ? s0 + 4 : s0;
    const int enext0 = load_scalar_i32(ex32, sn / 2), enext1 = load_scalar_i32(ex32, sn / 2 + 1);
    stage(s0, std::integral_constant<int, 0>{});
    stage(s0 + 1, std::integral_constant<int, 1>{});
    stage(s0 + 2, std::integral_constant<int, 2>{});
    stage(s0 + 3, std::integral_constant<int, 3>{});
    ecur0 = enext0;
    ecur1 = enext1;
  }
  const float fin = ldexpf(dp * 16777216.0f, -ep);
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (mt >= mtiles) break;
      const int m = 16 * mt + 4 * q + r;
      if (m < nrows) a.y[(size_t)(row0 + m) * a.H + n] = acc[mt][r] * fin;
    }
}

// down for routed items with Q4_K down weights: software-pipelined like
// k_grouped_down_q2k (same grid, h staging, weight ring and barriers).  A
// Q4_K block (fp16 d and dmin, twelve bytes of the 6-bit scales sc_j and mins
// m_j of its eight 32-column groups, 128 code bytes) spans two 128-column
// stages: stage half hf holds code chunks 2hf and 2hf + 1, and byte l of
// chunk c carries column 64c + l in its low nibble (group 2c) and column
// 64c + 32 + l in its high nibble (group 2c + 1).  Lane quarter q takes bytes
// 8q .. 8q+7 of each chunk: for each of the stage's four groups the B
// fragment of one f16 16x16x32 MFMA step (columns 32j + 8q .. +7 of the
// stage), with the group's scale folded in:
//   B = q * sc as a binary16 subnormal (q * sc <= 945: q sc 2^-24, exact),
//   A = the SwiGLU rows as binary16 high and low parts (two MFMAs).
// The accumulators hold the sum in units of the current block's d and of
// 2^-e, e the binary16 exponent of the current 64-column chunk (the grouped
// gate/up kernels store one per row and 64-feature range, the same for all
// rows of an item): a new block rescales them by the ratio of the d, a new
// exponent by a power of two (exact).  The mins, per chunk: one f16 16x16x16
// MFMA pair (hi, lo) of the stage's eight 16-feature sums of h against the
// chunk's mins (m_j as binary16 subnormals, in quarter c only: its K slots
// hold the chunk's four sums), scaled by dmin / d.
struct Q4kSub {
  uint4 hd;                // the block header: d | dmin << 16, scale and min bytes
  uint32_t c0, c1, c2, c3;  // the lane's code bytes of chunks 2hf and 2hf + 1
};

__device__ inline void q4k_sub_load(const uint8_t* __restrict__ row, int s, int q, Q4kSub& o) {
  const uint8_t* blk = row + kQ4kBytes * (s >> 1);
  const int hf = s & 1;
  o.hd = *(const uint4*)blk;
  const uint2 a = *(const uint2*)(blk + 16 + 64 * hf + 8 * q);
  const uint2 b = *(const uint2*)(blk + 16 + 64 * hf + 32 + 8 * q);
  o.c0 = a.x;
  o.c1 = a.y;
  o.c2 = b.x;
  o.c3 = b.y;
}

// MT = 1: the small items (at most 16 rows, listed first); MT = 4: the rest.
template <int MT>
__global__ __launch_bounds__(kDW * 64) void k_grouped_down_q4k(GroupArgs a) {
  constexpr int kRows = 16 * MT;
  constexpr int kHC = kRows * 32;                          // h chunks of a stage (hi, lo)
  constexpr int kHJ = (kHC + kDW * 64 - 1) / (kDW * 64);  // per thread
  constexpr int kSC = kRows * 2;                           // sum chunks (hi, lo)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ u32x4_t ht[2][kHC];  // row m: [hi 16 chunks][lo 16 chunks], chunk c at c ^ (m & 15)
  __shared__ u32x4_t st[2][kSC];  // row m: [8 sums hi][8 sums lo]
  const int n_small = a.n_items[1];
  const int item = (MT == 1 ? 0 : n_small) + (int)blockIdx.y;
  if (item >= (MT == 1 ? n_small : a.n_items[0])) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  if (e >= a.E) return;  // shared-expert items run in k_grouped_down
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  const int n = blockIdx.x * kDNF + 16 * w + (lane & 15);
  const int rowbytes = (a.I / 256) * kQ4kBytes;
  const uint8_t* drow = a.down + ((size_t)e * a.H + n) * rowbytes;
  const int nst = a.I / 128;  // a multiple of 4
  const int mtiles = (nrows + 15) >> 4;
  // h tile loads as in k_grouped_down_q2k: chunk c = tid + 512 j -> row
  // c >> 5, part (c >> 4) & 1, chunk c & 15; sum chunk cs = tid mod 2 kRows.
  // Rows past the item repeat row 0 (never stored).
  struct HV {
    u32x4_t v[kHJ];
    u32x4_t sm;
  };
  const uint16_t* hsrc[kHJ];
#pragma unroll
  for (int j = 0; j < kHJ; j++) {
    const int c = (tid + kDW * 64 * j) & (kHC - 1), m = c >> 5;
    const size_t r = (size_t)(row0 + (m < nrows ? m : 0));
    hsrc[j] = ((c >> 4) & 1 ? a.hl : a.hh) + r * a.I + 8 * (c & 15);
  }
  const int cs = tid & (kSC - 1), ms = cs >> 1;
  const uint16_t* ssrc = ((cs & 1) ? a.hsl : a.hsh) + (size_t)(row0 + (ms < nrows ? ms : 0)) * (a.I / 16);
  auto h_load = [&](int s) {
    HV r;
#pragma unroll
    for (int j = 0; j < kHJ; j++) r.v[j] = *(const u32x4_t*)(hsrc[j] + 128 * s);
    r.sm = *(const u32x4_t*)(ssrc + 8 * s);
    return r;
  };
  auto h_store = [&](int buf, const HV& h) {
#pragma unroll
    for (int j = 0; j < kHJ; j++) {
      const int c = (tid + kDW * 64 * j) & (kHC - 1), m = c >> 5;
      ht[buf][m * 32 + (c & 16) + ((c & 15) ^ (m & 15))] = h.v[j];
    }
    st[buf][cs] = h.sm;
  };
  // in-order returns: weights of stages 0 and 1, h of stages 0 and 1, then
  // the weights of stage 2
  Q4kSub W[4];
  q4k_sub_load(drow, 0, q, W[0]);
  q4k_sub_load(drow, 1, q, W[1]);
  __builtin_amdgcn_sched_barrier(0);
  HV H0 = h_load(0), H1 = h_load(1);
  __builtin_amdgcn_sched_barrier(0);
  q4k_sub_load(drow, 2, q, W[2]);
  __builtin_amdgcn_sched_barrier(0);
  h_store(0, H0);
  __syncthreads();

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float dp = 1.0f;  // d of the current block
  // exponent bytes of the item's first row (64-feature range r at byte r),
  // read through the scalar cache four stages ahead
  const int32_t* ex32 = (const int32_t*)(a.hexp + (size_t)row0 * (a.I / 64));
  int ecur0 = load_scalar_i32(ex32, 0), ecur1 = load_scalar_i32(ex32, 1);
  int ep = (int8_t)(ecur0 & 0xFF);  // exponent the accumulators are in
  auto stage = [&](int s, auto Rc) {
    constexpr int R = decltype(Rc)::value;
    constexpr int hf = R & 1;
    if constexpr ((R & 1) == 0) H0 = h_load(min(s + 2, nst - 1));
    else H1 = h_load(min(s + 2, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    q4k_sub_load(drow, s + 3 < nst ? s + 3 : s - 1, q, W[(R + 3) & 3]);
    __builtin_amdgcn_sched_barrier(0);
    const Q4kSub& cw = W[R];
    const float dv = f16_bits_to_f32(cw.hd.x & 0xFFFFu);
    const float d = dv != 0.0f ? dv : 1.0f;
    const float rd = __builtin_amdgcn_rcpf(d);  // within 1 ulp
    const float fmin = f16_bits_to_f32(cw.hd.x >> 16) * rd;
    if constexpr (hf == 0) {  // a block starts: sums in units of its d
      const float r = dp * rd;
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[mt] *= r;
      dp = d;
    }
    const u32x4_t* hb = ht[R & 1];
    const u32x4_t* sb = st[R & 1];
    const uint32_t ew = R < 2 ? (uint32_t)ecur0 : (uint32_t)ecur1;
#pragma unroll
    for (int c = 0; c < 2; c++) {
      // the chunk's exponent: 64-feature range 2s + c
      const int es = (int8_t)((ew >> (16 * (R & 1) + 8 * c)) & 0xFFu), de = es - ep;
      ep = es;
      if (de != 0) {
        const float r = ldexpf(1.0f, de);
#pragma unroll
        for (int mt = 0; mt < MT; mt++) acc[mt] *= r;
      }
      // code bytes in 16-bit lanes: (b0, b1), (b2, b3), (b4, b5), (b6, b7)
      const uint32_t cx = c ? cw.c2 : cw.c0, cy = c ? cw.c3 : cw.c1;
      const uint32_t P[4] = {vperm(0u, cx, 0x0C010C00u), vperm(0u, cx, 0x0C030C02u),
                             vperm(0u, cy, 0x0C010C00u), vperm(0u, cy, 0x0C030C02u)};
#pragma unroll
      for (int hi = 0; hi < 2; hi++) {
        const int jl = 2 * c + hi;  // group of the stage, 4 hf + jl of the block
        int sc, mn;
        q4k_scale_min(cw.hd, 4 * hf + jl, sc, mn);
        const uint32_t scm = dv != 0.0f ? (uint32_t)sc : 0u;
        // low nibbles: q sc in each 16-bit lane; high nibbles: 16 q sc
        // (below 2^14), shifted down by 4.  The unsigned 24-bit multiply:
        // the masked high nibbles reach bit 23, a sign bit to the signed one
        uint32_t bw[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
          bw[i] = hi ? __umul24(P[i] & 0x00F000F0u, scm) >> 4 : __umul24(P[i] & 0x000F000Fu, scm);
        const f16x8_t bf = __builtin_bit_cast(f16x8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          if (MT > 1 && mt >= mtiles) break;
          const int m = 16 * mt + (lane & 15);
          const int ci = (4 * jl + q) ^ (m & 15);
          const f16x8_t ahi = __builtin_bit_cast(f16x8_t, hb[m * 32 + ci]);
          const f16x8_t alo = __builtin_bit_cast(f16x8_t, hb[m * 32 + 16 + ci]);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bf, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bf, acc[mt], 0, 0, 0);
        }
      }
      // the chunk's mins: sums 4c .. 4c+3 of the stage (quarter c's K slots;
      // sums 4c, 4c+1 in group 2c, 4c+2, 4c+3 in group 2c+1)
      {
        int scx, m0, m1;
        q4k_scale_min(cw.hd, 4 * hf + 2 * c, scx, m0);
        q4k_scale_min(cw.hd, 4 * hf + 2 * c + 1, scx, m1);
        const uint32_t w0 = q == c ? (uint32_t)m0 * 0x00010001u : 0u;
        const uint32_t w1 = q == c ? (uint32_t)m1 * 0x00010001u : 0u;
        const f16x4_t bm = __builtin_bit_cast(f16x4_t, make_uint2(w0, w1));
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          if (MT > 1 && mt >= mtiles) break;
          const int m = 16 * mt + (lane & 15);
          const uint2* sp = (const uint2*)&sb[2 * m];
          const uint2 shi = sp[q & 1], slo = sp[2 + (q & 1)];
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, shi), bm, z, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, slo), bm, t, 0, 0, 0);
          acc[mt] -= fmin * t;
        }
      }
    }
    // h of stage s + 1 into the other buffers (after the last stage: unused)
    if constexpr ((R & 1) == 0) h_store(1, H1);
    else h_store(0, H0);
    __syncthreads();
  };
  for (int s0 = 0; s0 < nst; s0 += 4) {
    const int sn = s0 + 4 < nst ? s0 + 4 : s0;
    const int enext0 = load_scalar_i32(ex32, sn / 2), enext1 = load_scalar_i32(ex32, sn / 2 + 1);
    stage(s0, std::integral_constant<int, 0>{});
    stage(s0 + 1, std::integral_constant<int, 1>{});
    stage(s0 + 2, std::integral_constant<int, 2>{});
    stage(s0 + 3, std::integral_constant<int, 3>{});
    ecur0 = enext0;
    ecur1 = enext1;
  }
  const float fin = ldexpf(dp * 16777216.0f, -ep);
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (mt >= mtiles) break;
      const int m = 16 * mt + 4 * q + r;
      if (m < nrows) a.y[(size_t)(row0 + m) * a.H + n] = acc[mt][r] * fin;
    }
}

// out[t] = sum_k w[t][k] y[inv[t*K+k]] (+ the shared row) (+ residual), fixed
// order.  The shared row (with_shared) is y[T*K + t], or with ksplit > 1 the
// sum of its K shares in part ([ksplit][T][H]) in share order.  Four
// consecutive columns per thread (16-byte loads of y); H is a multiple of 256,
// so a wave covers 256 columns of one token and reads the token's rows and
// gates through the scalar cache.  vec_out: out and residual are 16-byte
// aligned and take 16-byte accesses too.
__global__ void k_grouped_combine(const float* y, const int32_t* inv, const float* wts, int T, int K,
                                  int H, int with_shared, float* out, float* residual,
                                  const float* part, int ksplit, int vec_out) {
  const size_t idx = 4 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (idx >= (size_t)T * H) return;  // whole waves (T * H is a multiple of 256)
  const int t = __builtin_amdgcn_readfirstlane((int)(idx / H)), c = (int)(idx % H);
  float4 sh = make_float4(0.f, 0.f, 0.f, 0.f);
  if (with_shared) {
    if (ksplit == 1) {
      sh = *(const float4*)(y + ((size_t)T * K + t) * H + c);
    } else {
      for (int z = 0; z < ksplit; z++) {
        const float4 v = *(const float4*)(part + (size_t)z * T * H + idx);
        sh.x += v.x;
        sh.y += v.y;
        sh.z += v.z;
        sh.w += v.w;
      }
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < K; k++) {
    const float wk = __int_as_float(load_scalar_i32((const int32_t*)wts, t * K + k));
    const int r = load_scalar_i32(inv, t * K + k);
    const float4 v = *(const float4*)(y + (size_t)r * H + c);
    acc.x = fmaf(wk, v.x, acc.x);
    acc.y = fmaf(wk, v.y, acc.y);
    acc.z = fmaf(wk, v.z, acc.z);
    acc.w = fmaf(wk, v.w, acc.w);
  }
  if (with_shared) {
    acc.x += sh.x;
    acc.y += sh.y;
    acc.z += sh.z;
    acc.w += sh.w;
  }
  float* dst = residual ? residual : out;
  if (vec_out) {
    float4 o = acc;
    if (residual) {
      const float4 r = *(const float4*)(residual + idx);
      o = make_float4(r.x + acc.x, r.y + acc.y, r.z + acc.z, r.w + acc.w);
    }
    *(float4*)(dst + idx) = o;
  } else {
    const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int u = 0; u < 4; u++) {
      if (residual) residual[idx + u] += a4[u];
      else out[idx + u] = a4[u];
    }
  }
}

// Importance statistics of the routed experts' inputs (DS4C2 =
// qiita.com/yoshiyakato/items/4678be0e7860ddb444ec, sections 5 and 7): per
// expert and input column, the sum over the expert's pairs of x^2 (gate/up
// input) and of (w h)^2 (down input: the SwiGLU row after the routing
// weight), accumulated into fp32 [E][H] and [E][I].  Grid (E, ceil(max(H,
// I)/64)), 256 threads: lane L of wave j owns column 64b + L and sums the
// expert's pairs j, j+4, j+8, .. of its sorted list in fp64 (sixteen pair
// ids per vector load, the sixteen pairs' loads issued before their sums);
// the four wave sums are added in wave order and once into the output, so
// the result depends only on the call's inputs.  h: fp32 rows indexed by
// pair (h_stride apart), or binary16 high + low parts indexed by sorted row
// (the grouped path).
struct ImxArgs {
  const void* x;
  int x_dt, H, I, K;
  const int32_t* offsets;
  const int32_t* perm;
  const float* wts;
  const float* h32;
  int h_stride;
  const uint16_t* hh;
  const uint16_t* hl;
  const int8_t* hexp;   // with hh/hl: the exponent of each row's 64-feature range
  float* gu;
  float* dn;
};

// XF32: x is fp32 (else bf16); HF16: h as binary16 parts by sorted row
// (else fp32 by pair).  Branch-free inner loop, so a batch's loads issue
// together.
template <bool XF32, bool HF16>
__global__ __launch_bounds__(256) void k_imatrix(ImxArgs a) {
  __shared__ double part[2][4][64];
  const int e = blockIdx.x, lane = threadIdx.x & 63;
  const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = blockIdx.y * 64 + lane;
  const int r0 = __builtin_amdgcn_readfirstlane(a.offsets[e]);
  const int n = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]) - r0;
  if (n <= 0) return;
  const bool cg = c < a.H, cd = c < a.I;
  const int cgc = cg ? c : 0, cdc = cd ? c : 0;  // loads stay in bounds
  constexpr int U = 16;
  double sg = 0.0, sd = 0.0;
  for (int i0 = j; i0 < n; i0 += 4 * U) {
    // the batch's pair ids: one vector load (lane u < U), then broadcast
    const int il = i0 + 4 * (lane & (U - 1));
    const int pl = a.perm[r0 + (il < n ? il : n - 1)];
    float xv[U], hv[U], lv[U], wv[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int i = i0 + 4 * u;
      const int r = r0 + (i < n ? i : n - 1);  // past the end: a repeat, weighted 0
      const int p = __builtin_amdgcn_readlane(pl, u), t = p / a.K;
      const size_t xi = (size_t)t * a.H + cgc;
      if constexpr (XF32) xv[u] = ((const float*)a.x)[xi];
      else xv[u] = bf16_bits_to_f32(((const uint16_t*)a.x)[xi]);
      if constexpr (HF16) {
        const size_t hi = (size_t)r * a.I + cdc;
        const int ex = a.hexp[(size_t)r * (a.I / 64) + cdc / 64];
        hv[u] = ldexpf(f16_bits_to_f32(a.hh[hi]), -ex);
        lv[u] = ldexpf(f16_bits_to_f32(a.hl[hi]), -ex);
      } else {
        hv[u] = a.h32[(size_t)p * a.h_stride + cdc];
        lv[u] = 0.0f;
      }
      wv[u] = i < n ? a.wts[p] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const double x = (double)xv[u];
      sg += i0 + 4 * u < n ? x * x : 0.0;
      const double v = (double)wv[u] * ((double)hv[u] + (double)lv[u]);
      sd += v * v;
    }
  }
  part[0][j][lane] = sg;
  part[1][j][lane] = sd;
  __syncthreads();
  if (j == 0) {
    const double tg = ((part[0][0][lane] + part[0][1][lane]) + part[0][2][lane]) + part[0][3][lane];
    const double td = ((part[1][0][lane] + part[1][1][lane]) + part[1][2][lane]) + part[1][3][lane];
    if (cg) a.gu[(size_t)e * a.H + c] += (float)tg;
    if (cd) a.dn[(size_t)e * a.I + c] += (float)td;
  }
}

// gate/up + SwiGLU for routed items with Q4_K gate and up.  Grid
// (I / 64, items), 256 threads; wave w owns features n0 + 16w .. +15.  K
// runs in 128-column stages (half a block, four groups); a stage's weights
// (the block header and the code bytes of its two chunk pairs) are requested
// before its x tile (binary16, staged in LDS with the swizzle of
// k_grouped_gateup) is written, so the two loads overlap.
__global__ __launch_bounds__(256, 3) void k_grouped_gateup_q4k(GroupArgs a) {
  __shared__ uint4 xt[2][kMC * 16];  // x of stages s (read) and s + 1 (written)
  __shared__ int tok[kMC];
  const int item = grid_item(a);
  if (item >= *a.n_items) return;
  const int e = a.items[3 * item], row0 = a.items[3 * item + 1], nrows = a.items[3 * item + 2];
  if (e == a.E) return;  // the shared expert runs in its own kernels
  const int n0 = blockIdx.x * kNT;
  if (n0 >= a.I) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = lane >> 4;
  uint32_t xe[4];  // the rows' x exponents, for the epilogue (requested first)
  load_row_xexp<4>(a, row0, q, xe);
  const int n = n0 + 16 * w + (lane & 15);
  const int nb = a.H / 256, nst = 2 * nb;
  if (tid < kMC) tok[tid] = tid < nrows ? row_token(a, row0 + tid) : -1;
  const size_t rowg = (size_t)e * a.I + n;
  const uint8_t* G = a.gate + rowg * nb * kQ4kBytes;
  const uint8_t* U = a.up + rowg * nb * kQ4kBytes;
  const int mtiles = (nrows + 15) >> 4;
  f32x4_t accg[4], accu[4];
  for (int mt = 0; mt < 4; mt++) accg[mt] = accu[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f16x8_t ones = __builtin_bit_cast(f16x8_t, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
  // A stage is half a block (128 columns): the block header (d, dmin, scales)
  // and the lane's two code chunks, for gate and up.  Stage s + 1's weights
  // and x are requested while stage s is multiplied; x alternates between
  // the two LDS buffers, one barrier per stage.
  struct Q4kW {
    uint4 hg, hu;
    uint2 cg[2], cu[2];
  };
  auto wload = [&](int kh, Q4kW& W) {
    const int kb = kh >> 1, hf = kh & 1;
    const uint8_t* bg = G + kb * kQ4kBytes;
    const uint8_t* bu = U + kb * kQ4kBytes;
    W.hg = *(const uint4*)bg;
    W.hu = *(const uint4*)bu;
#pragma unroll
    for (int c = 0; c < 2; c++) {  // code chunk 2hf + c: groups 4hf + 2c (low), + 1 (high)
      W.cg[c] = *(const uint2*)(bg + 16 + 32 * (2 * hf + c) + 8 * q);
      W.cu[c] = *(const uint2*)(bu + 16 + 32 * (2 * hf + c) + 8 * q);
    }
  };
  // x chunk c = tid + 256 i (i < 4): row c >> 4, 16-byte column chunk c & 15;
  // rows past the item load nothing and store zeros
  auto xload = [&](int kh, uint4 (&xv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int c = tid + 256 * i, m = c >> 4, ch = c & 15;
      xv[i] = m < nrows ? ((const uint4*)(a.x16 + (size_t)tok[m] * a.H + 128 * kh))[ch]
                        : make_uint4(0, 0, 0, 0);
    }
  };
  auto xstore = [&](int buf, const uint4 (&xv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int c = tid + 256 * i, m = c >> 4, ch = c & 15;
      xt[buf][m * 16 + (ch ^ (m & 15))] = xv[i];
    }
  };
  // stage kh = 2 kb + HF (HF a constant, so the sub-block of every scale and
  // min is known at compile time); Wc holds its weights, Wn receives the next
  auto stage = [&](int kh, auto HFc, const Q4kW& Wc, Q4kW& Wn) {
    constexpr int hf = decltype(HFc)::value;
    const bool more = kh + 1 < nst;
    uint4 xn[4];
    if (more) {
      xload(kh + 1, xn);
      wload(kh + 1, Wn);
    }
    const uint4* xb = xt[hf];
    const float dg = f16_bits_to_f32(Wc.hg.x & 0xFFFFu), mg = f16_bits_to_f32(Wc.hg.x >> 16);
    const float du = f16_bits_to_f32(Wc.hu.x & 0xFFFFu), mu = f16_bits_to_f32(Wc.hu.x >> 16);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      const uint4 pg = q4k_pairs(Wc.cg[c]), pu = q4k_pairs(Wc.cu[c]);
#pragma unroll
      for (int hi = 0; hi < 2; hi++) {
        const int gi = 2 * c + hi, j = 4 * hf + gi;
        int scg, mng, scu, mnu;
        q4k_scale_min(Wc.hg, j, scg, mng);
        q4k_scale_min(Wc.hu, j, scu, mnu);
        const float unit = hi ? 1048576.0f : 16777216.0f;  // 2^24 / 16^hi
        const float sgm = dg * (float)scg * unit, sgn = mg * (float)mng;
        const float sum = du * (float)scu * unit, sun = mu * (float)mnu;
        const f16x8_t fg = q4k_frag(pg, hi), fu = q4k_frag(pu, hi);
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          if (mt >= mtiles) break;
          const int m = 16 * mt + (lane & 15);
          const f16x8_t af = __builtin_bit_cast(f16x8_t, xb[m * 16 + ((4 * gi + q) ^ (m & 15))]);
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          const f32x4_t tg = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fg, z, 0, 0, 0);
          const f32x4_t tu = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fu, z, 0, 0, 0);
          const f32x4_t t1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, ones, z, 0, 0, 0);
          accg[mt] += sgm * tg - sgn * t1;
          accu[mt] += sum * tu - sun * t1;
        }
      }
    }
    if (more) xstore(hf ^ 1, xn);
    __syncthreads();
  };
  Q4kW WA, WB;
  wload(0, WA);
  __syncthreads();  // tok
  {
    uint4 xv[4];
    xload(0, xv);
    xstore(0, xv);
  }
  __syncthreads();
  for (int kh = 0; kh < nst; kh += 2) {  // nst is even
    stage(kh, std::integral_constant<int, 0>{}, WA, WB);
    stage(kh + 1, std::integral_constant<int, 1>{}, WB, WA);
  }
  swiglu_store(a, row0, nrows, mtiles, n, q, accg, accu, n0, kNT, xe, (uint32_t*)xt[0]);
}

// The grouped kernels need bf16 x, 256-multiple shapes and formats they know
// (any token count; after the few-token matvec kernels they also run a shared
// expert the per-token shared kernels do not take).
inline bool grouped_eligible(const ds4moe_shape& s, const ds4moe_experts& ex,
                             const ds4moe_experts* sh, const void* x, int32_t x_dt, int32_t T) {
  auto gu_ok = [](int qt) { return qt == DS4MOE_IQ2_XXS || qt == DS4MOE_Q8_0; };
  auto dn_ok = [](int qt) { return qt == DS4MOE_Q2_K || qt == DS4MOE_Q8_0 || qt == DS4MOE_Q4_K; };
  if (x_dt != DS4MOE_BF16 || ((uintptr_t)x % 16) != 0 || s.hidden % 256 || ex.inter % 256) return false;
  // routed gate/up: IQ2_XXS or Q8_0 each, or both Q4_K
  const bool gu_q4k = ex.gate_qtype == DS4MOE_Q4_K && ex.up_qtype == DS4MOE_Q4_K;
  if ((!gu_q4k && (!gu_ok(ex.gate_qtype) || !gu_ok(ex.up_qtype))) || !dn_ok(ex.down_qtype))
    return false;
  if (((uintptr_t)ex.gate | (uintptr_t)ex.up | (uintptr_t)ex.down) % 16) return false;
  if (sh) {
    if (!gu_ok(sh->gate_qtype) || !gu_ok(sh->up_qtype) || !dn_ok(sh->down_qtype)) return false;
    if (sh->inter % 256 || ((uintptr_t)sh->gate | (uintptr_t)sh->up | (uintptr_t)sh->down) % 16) return false;
  }
  return T >= 1;
}

}  // namespace ds4
