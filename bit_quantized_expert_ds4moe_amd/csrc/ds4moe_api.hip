// ds4moe_api.hip -- C ABI of libds4moe (declared in include/ds4moe.h):
// argument checks, workspace layout and kernel dispatch.  Built as one
// translation unit with the kernel sources.
#include <hip/hip_ext.h>
#include <string.h>

#include <mutex>

#include "dev_common.h"
#include "route.hip"
#include "ffn_b1.hip"
#include "ffn_q4k.hip"
#include "ffn_shared.hip"
#include "ffn_generic.hip"
#include "grouped.hip"
#include "encode.hip"

#define DS4_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace ds4;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Few-token calls use the streaming matvec kernels (in layer calls with the
// IQ2_XXS gate/up reading each distinct expert once, otherwise one grid row
// per token), which beat the grouped kernels up to kB1MaxTokensIq2 tokens of
// correlated decode with IQ2_XXS gate/up and Q2_K down (config-2 layer call,
// us: 9 tokens 132 vs 152, 10 tokens 143 vs 155, 11 tokens equal) and up to
// kB1MaxTokens with the other fast-path formats (Q4_K, not re-measured).
constexpr int kSharedB1MaxTokens = 2;  // shared expert by per-token matvecs up to here,
// then up to kSharedFewMaxTokens (on the matvec path) by matvecs that read its
// weights once for every token (3 tokens: 66.2 vs 67.3 us per layer call,
// 4: 80.5 vs 83.4; 2: 50.6 vs 50.0); beyond, by the grouped kernels
constexpr int kSharedFewMaxTokens = 10;
constexpr int kFuseSelMaxTokens = 4;  // layer calls: selection fused into gate/up up to here
// Above this many tokens the batch-1 down stages the SwiGLU vectors in LDS.
constexpr int kDnStageMinTokens = 4;
constexpr int kB1MaxTokens = 13;
constexpr int kB1MaxTokensIq2 = 10;
constexpr int kB1MaxTokensIq2Ids = 8;  // the same with caller-given ids (one grid row per token:
// 8 tokens 145 vs 149 us per call, 9 tokens 158 vs 151)
// Layer calls from this many tokens (selection kernel, no fused selection)
// read each distinct IQ2_XXS expert once in gate/up (k_gateup_few).
constexpr int kFewMinT = 2;
constexpr int kSharedSplitG = 16;  // K shares of a shared expert's gate/up in calls of few tokens (<= kMaxSplit)
constexpr int kSharedSplitD = 4;   // and of its down
constexpr int kSharedSplitMaxT = 64;  // "few": one work item of shared rows

// Byte offsets of the workspace regions for (shape, n_tok).
struct Layout {
  size_t status, kbuf, ids, wts, xn, x16, perm, h, y, hb, part, xexp, hexp, total;
};

Layout layout_for(const ds4moe_shape& s, int32_t T) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o = align_up(o + bytes, 256);
    return r;
  };
  const size_t E = (size_t)s.n_expert, K = (size_t)s.top_k, H = (size_t)s.hidden,
               I = (size_t)s.inter, t = (size_t)T;
  const size_t np = t * K + t;  // routed pairs + shared-expert rows
  L.status = take(256);
  L.kbuf = take(t * E * 16);
  L.ids = take(t * K * 4);
  L.wts = take(t * K * 4);
  L.xn = take(t * H * 2);
  L.x16 = take(t * H * 2);
  L.perm = take((E + (E + 1) + 2 * t * K + 3 * (size_t)max_items_upto((int)E, (int)K, (int)t) + 64) * 4);
  L.h = take(np * I * 4);
  L.y = take(np * H * 4);
  L.hb = take(np * I * 2);
  // K shares of a shared expert in few-token calls
  L.part = take(t <= (size_t)kSharedSplitMaxT ? (size_t)kSharedSplitG * t * (2 * I > H ? 2 * I : H) * 4 : 0);
  // binary16 exponents of the grouped path: x's per sorted row (the token's;
  // 64 rows of padding read by the last tiles), the SwiGLU rows' per row and
  // 64-feature range
  L.xexp = take((t * K + 64) * 4);
  L.hexp = take(np * ((I + 63) / 64));
  L.total = o;
  return L;
}

bool shape_ok(const ds4moe_shape* s) {
  return s && s->hidden > 0 && s->hidden % 256 == 0 && s->inter > 0 && s->inter % 32 == 0 &&
         s->n_expert >= 1 && s->n_expert <= 256 && s->top_k >= 1 && s->top_k <= s->n_expert &&
         s->top_k <= 64;
}

bool qtype_ok(int32_t q) {
  return q == DS4MOE_Q2_K || q == DS4MOE_IQ2_XXS || q == DS4MOE_Q8_0 || q == DS4MOE_Q4_K;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool experts_ok(const ds4moe_experts* ex, int32_t H) {
  if (!ex || !ex->gate || !ex->up || !ex->down) return false;
  if (!qtype_ok(ex->gate_qtype) || !qtype_ok(ex->up_qtype) || !qtype_ok(ex->down_qtype)) return false;
  if (ex->inter <= 0 || ex->inter % 32 != 0 || H % 256 != 0) return false;
  bool need_grid = ex->gate_qtype == DS4MOE_IQ2_XXS || ex->up_qtype == DS4MOE_IQ2_XXS ||
                   ex->down_qtype == DS4MOE_IQ2_XXS;
  if (need_grid && !ex->grid) return false;
  return aligned(ex->gate, 4) && aligned(ex->up, 4) && aligned(ex->down, 4);
}

ds4moe_status launched() {
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_EDEVICE;
}

// Profiling events per kernel class (ds4moe_profile_events).  While a class
// scope is open, kernels are launched with hipExtLaunchKernelGGL so that the
// events take the execution timestamps of the kernels themselves: the start
// event the first kernel's start, the stop event the last kernel's end.
hipEvent_t g_prof[DS4MOE_K_CLASSES][2] = {};

struct ProfScope {
  static ProfScope* active;
  int cls;
  bool started = false;
  ProfScope* prev;
  bool on;  // a disabled scope leaves its kernels to the enclosing one
  ProfScope(int c, hipStream_t, bool enabled = true) : cls(c), prev(active), on(enabled) {
    if (on) active = this;
  }
  ~ProfScope() {
    if (on) active = prev;
  }
};
ProfScope* ProfScope::active = nullptr;

template <typename... P, typename... A>
void launch_k(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t shm, hipStream_t st,
              A... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (ProfScope* p = ProfScope::active) {
    e1 = g_prof[p->cls][1];
    if (!p->started) e0 = g_prof[p->cls][0];
    p->started = true;
  }
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, shm, st, e0, e1, 0u, static_cast<P>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, st, static_cast<P>(args)...);
}

inline ds4moe_status launch_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                    int32_t* offsets, int32_t* perm, int32_t* inv,
                                    uint32_t* status, hipStream_t st, int T = 0,
                                    int with_shared = 0, int32_t* items = nullptr,
                                    int32_t* n_items = nullptr) {
  if (n > kPermMax) return DS4MOE_EUNSUPPORTED;
  launch_k(k_permute, dim3(1), dim3(1024), 0, st, ids, n, E, counts, offsets, perm, inv, status,
           T, with_shared, items, n_items);
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_EDEVICE;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Permutation and work-item arrays in the workspace (the grouped path's, also
// built by the selection kernel for the few-token distinct-expert gate/up).
struct PermPtrs {
  int32_t *counts, *offsets, *perm, *inv, *items, *n_items;
};
PermPtrs perm_ptrs(const ds4moe_shape& s, int32_t T, void* ws, const Layout& L) {
  const int E = s.n_expert, TK = T * s.top_k;
  PermPtrs p;
  p.counts = at<int32_t>(ws, L.perm);
  p.offsets = p.counts + E;
  p.perm = p.offsets + E + 1;
  p.inv = p.perm + TK;
  p.items = p.inv + TK;
  p.n_items = p.items + 3 * max_items(E, TK, T, true);
  return p;
}

// ---- routing ---------------------------------------------------------------
// The scoring kernel's 16-byte column layout applies (hidden a multiple of
// 2048 up to 4096, f16 router, bf16 or normalised input, aligned rows).
bool route_vec(const ds4moe_shape& s, const ds4moe_router& r, const void* x, int32_t x_dt,
               const float* residual, const float* norm_w, const uint16_t* xn_out) {
  return s.hidden % 2048 == 0 && s.hidden <= 4096 && r.w_dtype == DS4MOE_F16 &&
         (norm_w || x_dt == DS4MOE_BF16) && ((uintptr_t)r.w % 16 == 0) &&
         (norm_w ? ((uintptr_t)residual % 16 == 0 && (uintptr_t)norm_w % 16 == 0 &&
                    (uintptr_t)xn_out % 16 == 0)
                 : (uintptr_t)x % 16 == 0);
}

ds4moe_status do_route(const ds4moe_shape& s, const ds4moe_router& r, const void* x, int32_t x_dt,
                       const float* residual, const float* norm_w, float eps, uint16_t* xn_out,
                       int32_t T, const int32_t* tok, int32_t* ids, float* wts, void* ws,
                       const Layout& L, hipStream_t st, bool select = true,
                       bool few_items = false, const SharedB1Args* shu = nullptr) {
  uint32_t* status = at<uint32_t>(ws, L.status);
  ProfScope prof(DS4MOE_K_ROUTE, st);
  if (r.tid2eid) {
    launch_k(k_route_hash, dim3((T + 255) / 256), dim3(256), 0, st, tok, r.tid2eid,
                       r.vocab, s.n_expert, s.top_k, T, s.routed_scale, ids, wts, status);
    return launched();
  }
  RouteArgs a{};
  a.x = x;
  a.x_dt = x_dt;
  a.residual = residual;
  a.norm_w = norm_w;
  a.eps = eps;
  a.xn_out = xn_out;
  a.W = r.w;
  a.w_dt = r.w_dtype;
  a.bias = r.bias;
  a.H = s.hidden;
  a.E = s.n_expert;
  a.K = s.top_k;
  a.T = T;
  a.scale = s.routed_scale;
  a.kbuf = at<float4>(ws, L.kbuf);
  a.ids = ids;
  a.wts = wts;
  a.status = status;
  // the selection kernel also lists the items (one workgroup, a wave per token)
  if (few_items && T * s.top_k <= kSelItemsMax && T <= 16) {
    const PermPtrs pp = perm_ptrs(s, T, ws, L);
    a.perm = pp.perm;
    a.items = pp.items;
    a.n_items = pp.n_items;
  }
  const bool vec = route_vec(s, r, x, x_dt, residual, norm_w, xn_out);
  const dim3 grid(s.n_expert, T);
  if (shu) {  // with the shared expert's gate/up (independent of the routing)
    const dim3 ug(s.n_expert + kI / 8, T);
    const bool few = T > kSharedB1MaxTokens;
    // (with norm_w the caller has checked vec and T <= kSharedB1MaxTokens)
    if (norm_w) launch_k(k_route_score_shared<true, false, true>, ug, dim3(256), 0, st, a, *shu, T);
    else if (vec && few) launch_k(k_route_score_shared<true, true, false>, ug, dim3(256), 0, st, a, *shu, T);
    else if (vec) launch_k(k_route_score_shared<true, false, false>, ug, dim3(256), 0, st, a, *shu, T);
    else if (few) launch_k(k_route_score_shared<false, true, false>, ug, dim3(256), 0, st, a, *shu, T);
    else launch_k(k_route_score_shared<false, false, false>, ug, dim3(256), 0, st, a, *shu, T);
  } else if (vec && norm_w)
    launch_k(k_route_score<true, true>, grid, dim3(256), 0, st, a);
  else if (vec)
    launch_k(k_route_score<false, true>, grid, dim3(256), 0, st, a);
  else if (norm_w)
    launch_k(k_route_score<true, false>, grid, dim3(256), 0, st, a);
  else
    launch_k(k_route_score<false, false>, grid, dim3(256), 0, st, a);
  ds4moe_status rc = launched();
  if (rc != DS4MOE_OK || !select) return rc;
  if (a.items) launch_k(k_route_select, dim3(1), dim3(64 * T), 0, st, a);
  else launch_k(k_route_select, dim3(T), dim3(64), 0, st, a);
  return launched();
}

// RMSNorm only (hash layers): one block per token writes xn.
// Hash routing done beside the RMSNorm (one launch for both in hash-routed
// layers): the arguments of route_hash_token, table == nullptr for none.
struct HashArgs {
  const int32_t* tok;
  const int32_t* table;
  int vocab, E, K;
  float scale;
  int32_t* ids;
  float* wts;
  uint32_t* status;
};

// RMSNorm of the residual stream to bf16 (used where routing does not fold it
// in, i.e. hash-routed layers).  One block per token; up to 4096 columns the
// loads of a thread are all issued before the first use.  With hs.table the
// block's last lane also routes its token by the table (the two do not depend
// on each other; the lookup's loads overlap the norm's).
__global__ __launch_bounds__(256) void k_rmsnorm_bf16(const float* residual, const float* w,
                                                     float eps, int H, uint16_t* xn, HashArgs hs) {
  __shared__ double sh[8];
  constexpr int kRegCols = 16;
  const int t = blockIdx.x, tid = threadIdx.x;
  auto route = [&]() {
    if (hs.table && tid == 255)
      route_hash_token(t, hs.tok, hs.table, hs.vocab, hs.E, hs.K, hs.scale, hs.ids, hs.wts, hs.status);
  };
  const float* r = residual + (size_t)t * H;
  double ss = 0.0, dummy = 0.0;
  if (H <= 256 * kRegCols) {
    float v[kRegCols], wv[kRegCols];
#pragma unroll
    for (int j = 0; j < kRegCols; j++) {
      const int c = tid + 256 * j;
      v[j] = c < H ? r[c] : 0.0f;
      wv[j] = c < H ? w[c] : 0.0f;
    }
    route();  // behind the norm's loads, which it waits for first
#pragma unroll
    for (int j = 0; j < kRegCols; j++) ss = fma((double)v[j], (double)v[j], ss);
    block_sum2(ss, dummy, sh);
    const double ns = 1.0 / sqrt(ss / (double)H + (double)eps);
    // results outside the normal bfloat16 range (rare) take the general
    // rounding in a separate pass, so the common loop has no call in it
    uint32_t bb[kRegCols];
    bool all_ok = true;
#pragma unroll
    for (int j = 0; j < kRegCols; j++) {
      bool ok;
      bb[j] = f64_to_bf16_bits_fast((double)v[j] * ns * (double)wv[j], ok);
      all_ok &= ok;
    }
    if (!all_ok)
      for (int j = 0; j < kRegCols; j++) {
        bool ok;
        (void)f64_to_bf16_bits_fast((double)v[j] * ns * (double)wv[j], ok);
        if (!ok) bb[j] = f64_to_bf16_bits_general((double)v[j] * ns * (double)wv[j]);
      }
#pragma unroll
    for (int j = 0; j < kRegCols; j++) {
      const int c = tid + 256 * j;
      if (c < H) xn[(size_t)t * H + c] = (uint16_t)bb[j];
    }
    return;
  }
  route();
  for (int c = tid; c < H; c += 256) {
    double v = (double)r[c];
    ss = fma(v, v, ss);
  }
  block_sum2(ss, dummy, sh);
  const double ns = 1.0 / sqrt(ss / (double)H + (double)eps);
  for (int c = tid; c < H; c += 256)
    xn[(size_t)t * H + c] = (uint16_t)f64_to_bf16_bits((double)r[c] * ns * (double)w[c]);
}

// ---- expert FFN dispatch ----------------------------------------------------
// Few tokens (up to kB1MaxTokensIq2 or kB1MaxTokens) with the V4-Flash expert shape and formats:
// the streaming matvec kernels, one grid row per token (the routed experts;
// a shared expert then runs through the grouped path, split along K).
bool fast_b1(const ds4moe_shape& s, const ds4moe_experts& ex, const void* x, int32_t x_dt,
             int32_t T, bool few_items = false) {
  // gate/up: both IQ2_XXS or both Q4_K; down: Q2_K or Q4_K
  const bool gu = (ex.gate_qtype == DS4MOE_IQ2_XXS && ex.up_qtype == DS4MOE_IQ2_XXS) ||
                  (ex.gate_qtype == DS4MOE_Q4_K && ex.up_qtype == DS4MOE_Q4_K);
  const bool dn = ex.down_qtype == DS4MOE_Q2_K || ex.down_qtype == DS4MOE_Q4_K;
  const bool iq2_q2k = ex.gate_qtype == DS4MOE_IQ2_XXS && ex.down_qtype == DS4MOE_Q2_K;
  const int tmax = iq2_q2k ? (few_items ? kB1MaxTokensIq2 : kB1MaxTokensIq2Ids) : kB1MaxTokens;
  return T >= 1 && T <= tmax && x_dt == DS4MOE_BF16 &&
         s.hidden == kH && s.inter == kI && ex.inter == kI &&
         s.top_k == 6 && gu && dn && aligned(x, 16) && aligned(ex.gate, 16) &&
         aligned(ex.up, 16) && aligned(ex.down, 16) && aligned(ex.grid, 8);
}

// Batch-1 fast path: gate/up (+ the top-6 selection when kbuf is given, in
// which case ids/wts are outputs) then down.
ds4moe_status launch_b1(const ds4moe_shape& s, const ds4moe_experts& ex, const void* x,
                        int32_t T, const int32_t* ids_in, const float4* kbuf, int32_t* ids,
                        const float* wts, float* out, float* residual, void* ws, const Layout& L,
                        hipStream_t st, const SharedB1Args* shb = nullptr,
                        const ds4moe_router* rt = nullptr, bool few_items = false,
                        bool sh_gu_done = false) {
  // one weight read for all tokens (kSharedB1MaxTokens < T <= kSharedFewMaxTokens)
  const bool sh_few = shb && T > kSharedB1MaxTokens && T <= kSharedFewMaxTokens;
  // the shared down as a seventh slot of the routed Q2_K down up to
  // kDnStageMinTokens tokens, also after the read-once gate/up (config-2 layer
  // call, 4 tokens: 75.3 / 74.0 -> 71.9 / 71.9 us); with more tokens, where
  // the routed down stages its rows in LDS, the read-once kernel of its own
  // (8 tokens: a seventh slot there took the down from 34.4 to 53.8 us)
  const bool sh_slot = shb && T <= kDnStageMinTokens && ex.down_qtype != DS4MOE_Q4_K;
  uint32_t* status = at<uint32_t>(ws, L.status);
  float* h = at<float>(ws, L.h);
  // the selection kernel listed one work item per distinct expert: the
  // IQ2_XXS gate/up reads each of them once for all its tokens
  const bool few = few_items && !kbuf && ids_in && ex.gate_qtype == DS4MOE_IQ2_XXS &&
                   ex.up_qtype == DS4MOE_IQ2_XXS;
  if (few) {
    const PermPtrs pp = perm_ptrs(s, T, ws, L);
    GateUpFewArgs f{};
    f.x = (const uint16_t*)x;
    f.gate = (const uint8_t*)ex.gate;
    f.up = (const uint8_t*)ex.up;
    f.grid = ex.grid;
    f.items = pp.items;
    f.n_items = pp.n_items;
    f.perm = pp.perm;
    f.h = h;
    const int TK = T * s.top_k;
    ProfScope prof(DS4MOE_K_GATEUP, st);
    launch_k(k_gateup_few, dim3(kI / kFewFeat, s.n_expert < TK ? s.n_expert : TK),
             dim3(kFewWaves * 64), 0, st, f);
  }
  GateUpB1Args g{};
  g.x = (const uint16_t*)x;
  g.gate = (const uint8_t*)ex.gate;
  g.up = (const uint8_t*)ex.up;
  g.grid = ex.grid;
  g.ids = ids_in;
  g.kbuf = kbuf;
  g.scale = s.routed_scale;
  g.ids_out = ids;
  g.wts_out = const_cast<float*>(wts);
  if (rt) {
    g.rw = rt->w;
    g.rw_dt = rt->w_dtype;
    g.rbias = rt->bias;
  }
  g.E = s.n_expert;
  g.h = h;
  g.status = status;
  if (!few) {
    ProfScope prof(DS4MOE_K_GATEUP, st);
    const bool q4 = ex.gate_qtype == DS4MOE_Q4_K;
    if (kbuf && q4)
      launch_k(k_gateup_q4k_b1<true>, dim3(kGuBlocks, T), dim3(kGuWaves * 64), 0, st, g);
    else if (kbuf)
      launch_k(k_gateup_b1<true>, dim3(kGuBlocks, T), dim3(kGuWaves * 64), 0, st, g);
    else if (q4)
      launch_k(k_gateup_q4k_b1<false>, dim3(kGuBlocks, T), dim3(kGuWaves * 64), 0, st, g);
    else
      launch_k(k_gateup_b1<false>, dim3(kGuBlocks, T), dim3(kGuWaves * 64), 0, st, g);
  }
  ds4moe_status rc = launched();
  if (rc != DS4MOE_OK) return rc;
  if (shb && !sh_gu_done) {  // the shared expert's gate/up; its down rides along with the routed one
    ProfScope prof(DS4MOE_K_OTHER, st);
    if (sh_few)
      launch_k(k_shared_gateup_q80_few, dim3(kI / 8, (T + kShFewTok - 1) / kShFewTok), dim3(256), 0,
               st, *shb, T);
    else launch_k(k_shared_gateup_q80_b1, dim3(kI / 8, T), dim3(256), 0, st, *shb);
    if ((rc = launched()) != DS4MOE_OK) return rc;
  }
  const int32_t* dids = kbuf ? ids : ids_in;
  const uint8_t* down = (const uint8_t*)ex.down;
  const dim3 dgrid(kH / kDnBlockRows, T);
  {
    ProfScope prof(DS4MOE_K_DOWN, st);
    if (ex.down_qtype == DS4MOE_Q4_K)
      launch_k(k_down_q4k_b1, dgrid, dim3(kDnThreads), 0, st, h, down, dids, wts, s.n_expert, out,
               residual, status);
    else if (sh_slot)
      launch_k(k_down_q2k_b1<true, false>, dgrid, dim3(kDnThreadsSh), 0, st, h, down, dids, wts,
               s.n_expert, out, residual, status, (const float*)shb->h, shb->down);
    else if (T > kDnStageMinTokens)
      launch_k(k_down_q2k_b1<false, true>, dgrid, dim3(kDnThreads), 0, st, h, down, dids, wts,
               s.n_expert, out, residual, status, (const float*)nullptr, (const uint8_t*)nullptr);
    else
      launch_k(k_down_q2k_b1<false, false>, dgrid, dim3(kDnThreads), 0, st, h, down, dids, wts,
               s.n_expert, out, residual, status, (const float*)nullptr, (const uint8_t*)nullptr);
  }
  if ((rc = launched()) != DS4MOE_OK) return rc;
  if (shb && !sh_slot) {  // the shared down on its own
    ProfScope prof(DS4MOE_K_OTHER, st);
    if (sh_few)
      launch_k(k_shared_down_q80_few, dim3(kH / 16, (T + kShFewTok - 1) / kShFewTok), dim3(256), 0,
               st, *shb, T);
    else launch_k(k_shared_down_q80_b1, dim3(kH / 16, T), dim3(256), 0, st, *shb);
    rc = launched();
  }
  return rc;
}

// Permutation for the caller's debug buffer (offsets[E+1], perm, inv).
ds4moe_status permute_dbg(const ds4moe_shape& s, int32_t T, const int32_t* ids, int32_t* perm_dbg,
                          void* ws, const Layout& L, hipStream_t st) {
  const int E = s.n_expert, TK = T * s.top_k;
  int32_t* counts = at<int32_t>(ws, L.perm);
  int32_t* offsets = counts + E;
  int32_t* perm = offsets + E + 1;
  int32_t* inv = perm + TK;
  ProfScope prof(DS4MOE_K_PERMUTE, st);
  ds4moe_status rc = launch_permute(ids, TK, E, counts, offsets, perm, inv,
                                    at<uint32_t>(ws, L.status), st);
  if (rc != DS4MOE_OK) return rc;
  if (hipMemcpyAsync(perm_dbg, offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToDevice, st) != hipSuccess ||
      hipMemcpyAsync(perm_dbg + E + 1, perm, sizeof(int32_t) * 2 * TK, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return DS4MOE_EDEVICE;
  return DS4MOE_OK;
}

// Importance statistics (ds4moe_expert_ffn_imatrix): launched by do_ffn once
// the routed SwiGLU rows exist and before anything reuses their memory.
struct ImxOut {
  float* gu;
  float* dn;
};

ds4moe_status launch_imatrix(const ds4moe_shape& s, const ImxOut& o, const void* x, int32_t x_dt,
                             int32_t T, const int32_t* ids, const float* wts, const float* h32,
                             int h_stride, const uint16_t* hh, const uint16_t* hl, bool have_perm,
                             void* ws, const Layout& L, hipStream_t st) {
  const int E = s.n_expert, TK = T * s.top_k;
  int32_t* counts = at<int32_t>(ws, L.perm);
  int32_t* offsets = counts + E;
  int32_t* perm = offsets + E + 1;
  int32_t* inv = perm + TK;
  ProfScope prof(DS4MOE_K_OTHER, st);
  if (!have_perm) {
    ds4moe_status rc = launch_permute(ids, TK, E, counts, offsets, perm, inv,
                                      at<uint32_t>(ws, L.status), st);
    if (rc != DS4MOE_OK) return rc;
  }
  ImxArgs a{};
  a.x = x;
  a.x_dt = x_dt;
  a.H = s.hidden;
  a.I = s.inter;
  a.K = s.top_k;
  a.offsets = offsets;
  a.perm = perm;
  a.wts = wts;
  a.h32 = h32;
  a.h_stride = h_stride;
  a.hh = hh;
  a.hl = hl;
  a.hexp = at<int8_t>(ws, L.hexp);
  a.gu = o.gu;
  a.dn = o.dn;
  const int cmax = s.hidden > s.inter ? s.hidden : s.inter;
  const dim3 grid(E, (cmax + 63) / 64), block(256);
  const bool xf32 = x_dt == DS4MOE_F32;
  if (xf32 && hh) launch_k(k_imatrix<true, true>, grid, block, 0, st, a);
  else if (xf32) launch_k(k_imatrix<true, false>, grid, block, 0, st, a);
  else if (hh) launch_k(k_imatrix<false, true>, grid, block, 0, st, a);
  else launch_k(k_imatrix<false, false>, grid, block, 0, st, a);
  return launched();
}

// Arguments of the shared expert's matvec kernels (its SwiGLU rows follow the
// routed rows in the workspace; its output is added to out or the residual).
SharedB1Args shared_args(const ds4moe_shape& s, const ds4moe_experts& sh, const void* x, int32_t T,
                         float* out, float* residual, void* ws, const Layout& L) {
  SharedB1Args sa{};
  sa.x = (const uint16_t*)x;
  sa.gate = (const uint8_t*)sh.gate;
  sa.up = (const uint8_t*)sh.up;
  sa.down = (const uint8_t*)sh.down;
  sa.h = at<float>(ws, L.h) + (size_t)T * s.top_k * s.inter;  // after the routed rows
  sa.out = residual ? residual : out;
  sa.status = at<uint32_t>(ws, L.status);
  return sa;
}

// do_ffn takes the few-token matvec path and runs the shared expert there by
// matvecs (the same tests as in do_ffn).
bool shared_by_matvecs(const ds4moe_shape& s, const ds4moe_experts& ex, const ds4moe_experts* sh,
                       const void* x, int32_t x_dt, int32_t T, bool few_items_only) {
  return sh && fast_b1(s, ex, x, x_dt, T, few_items_only) &&
         grouped_eligible(s, ex, sh, x, x_dt, T) && T <= kSharedFewMaxTokens &&
         shared_b1_ok(s, *sh, x, x_dt);
}

ds4moe_status do_ffn(const ds4moe_shape& s, const ds4moe_experts& ex, const ds4moe_experts* sh,
                     const void* x, int32_t x_dt, int32_t T, const int32_t* ids, const float* wts,
                     float* out, float* residual, int32_t* perm_dbg, void* ws, const Layout& L,
                     hipStream_t st, const ImxOut* imx = nullptr, const float4* kbuf_sel = nullptr,
                     const ds4moe_router* rt = nullptr, bool few_items = false,
                     bool sh_gu_done = false) {
  uint32_t* status = at<uint32_t>(ws, L.status);
  const bool b1 = fast_b1(s, ex, x, x_dt, T, few_items && !kbuf_sel) &&
                  (!sh || grouped_eligible(s, ex, sh, x, x_dt, T));
  if (b1) {
    // a Q8_0 shared expert runs inside launch_b1 as matvecs: per token up
    // to kSharedB1MaxTokens tokens, then one weight read for all tokens up to
    // kSharedFewMaxTokens; beyond, the grouped kernels below take it
    const bool shb1 = sh && T <= kSharedFewMaxTokens && shared_b1_ok(s, *sh, x, x_dt);
    const SharedB1Args sa = shb1 ? shared_args(s, *sh, x, T, out, residual, ws, L) : SharedB1Args{};
    // kbuf_sel: the top-K selection runs inside the gate/up kernel, which
    // writes ids and wts (workspace buffers then)
    ds4moe_status rc =
        kbuf_sel ? launch_b1(s, ex, x, T, nullptr, kbuf_sel, const_cast<int32_t*>(ids), wts, out,
                             residual, ws, L, st, shb1 ? &sa : nullptr, rt, false, sh_gu_done)
                 : launch_b1(s, ex, x, T, ids, nullptr, nullptr, wts, out, residual, ws, L, st,
                             shb1 ? &sa : nullptr, nullptr, few_items, sh_gu_done);
    if (rc == DS4MOE_OK && perm_dbg)  // the few-token path needs no permutation: make it for the caller
      rc = permute_dbg(s, T, ids, perm_dbg, ws, L, st);
    // h: fp32 [T][6][I] by pair; the shared expert's rows below reuse its memory
    if (rc == DS4MOE_OK && imx)
      rc = launch_imatrix(s, *imx, x, x_dt, T, ids, wts, at<float>(ws, L.h), s.inter, nullptr,
                          nullptr, false, ws, L, st);
    if (rc != DS4MOE_OK || !sh) return rc;
    if (shb1) return DS4MOE_OK;  // the shared expert ran inside launch_b1
  }
  if (b1 || (T > 1 && grouped_eligible(s, ex, sh, x, x_dt, T))) {
    // after the few-token path, the shared expert's kernels time as one class
    ProfScope shared_only(DS4MOE_K_OTHER, st, b1);
    const int E = s.n_expert, K = s.top_k, TK = T * K;
    int32_t* counts = at<int32_t>(ws, L.perm);
    int32_t* offsets = counts + E;
    int32_t* perm = offsets + E + 1;
    int32_t* inv = perm + TK;
    int32_t* items = inv + TK;
    // grid rows: every possible work item, or just the shared expert's rows
    const int mi = b1 ? (T + kMC - 1) / kMC : max_items(E, TK, T, sh != nullptr);
    int32_t* n_items = items + 3 * mi;
    ds4moe_status rc;
    {
      ProfScope prof(DS4MOE_K_PERMUTE, st, !b1);
      if (b1) {  // the routed experts are done: the shared expert's rows only
        launch_k(k_make_shared_items, dim3(1), dim3(64), 0, st, E, TK, T, items, n_items);
      } else {
        rc = launch_permute(ids, TK, E, counts, offsets, perm, inv, status, st, T, sh ? 1 : 0,
                            items, n_items);
        if (rc != DS4MOE_OK) return rc;
      }
    }
    if ((rc = launched()) != DS4MOE_OK) return rc;
    GroupArgs g{};
    g.H = s.hidden;
    g.I = ex.inter;
    g.E = E;
    g.K = K;
    g.T = T;
    g.x = (const uint16_t*)x;
    g.x16 = at<uint16_t>(ws, L.x16);
    g.perm = perm;
    g.items = items;
    g.n_items = n_items;
    g.gate = (const uint8_t*)ex.gate;
    g.up = (const uint8_t*)ex.up;
    g.down = (const uint8_t*)ex.down;
    g.qt_g = ex.gate_qtype;
    g.qt_u = ex.up_qtype;
    g.qt_d = ex.down_qtype;
    if (sh) {
      g.sh_gate = (const uint8_t*)sh->gate;
      g.sh_up = (const uint8_t*)sh->up;
      g.sh_down = (const uint8_t*)sh->down;
      g.sh_qt_g = sh->gate_qtype;
      g.sh_qt_u = sh->up_qtype;
      g.sh_qt_d = sh->down_qtype;
      g.sh_I = sh->inter;
    }
    g.grid = ex.grid ? ex.grid : (sh ? sh->grid : nullptr);
    {
      const size_t np = (size_t)TK + (size_t)T;
      uint16_t* hbase = at<uint16_t>(ws, L.h);
      g.hh = hbase;
      g.hl = hbase + np * (size_t)g.I;
      uint16_t* sbase = at<uint16_t>(ws, L.hb);
      g.hsh = sbase;
      g.hsl = sbase + np * (size_t)(g.I / 16);
    }
    g.xrexp = at<int8_t>(ws, L.xexp);
    g.hexp = at<int8_t>(ws, L.hexp);
    g.y = at<float>(ws, L.y);
    g.ksplit_g = g.ksplit_d = 1;
    g.part = at<float>(ws, L.part);
    if (sh && T <= kSharedSplitMaxT) {  // a single item of shared rows: spread it along K
      if ((g.H / 64) % kSharedSplitG == 0) g.ksplit_g = kSharedSplitG;
      if ((g.sh_I / 256) % kSharedSplitD == 0) g.ksplit_d = kSharedSplitD;
    }
    g.status = status;
    g.sh_tail = 0;
    // items of more than 16 rows only with 64-row pieces and more than 16 tokens
    const bool large = item_rows(T) > 16 && T > 16;
    // kernels that see only the shared expert's rows: grid rows over its
    // work items, the last ns of the list
    const int ns = (T + kMC - 1) / kMC;
    GroupArgs gs = g;
    gs.sh_tail = ns;
    const int imax = g.I > g.sh_I ? g.I : g.sh_I;
    {
      ProfScope prof(DS4MOE_K_GATEUP, st, !b1);
      const bool iq2 = iq2_grouped_fast(g);
      const bool q4k = q4k_grouped_gu(g);
      const bool q80 = sh && q80_shared_fast(g);
      if ((iq2 || q4k) && !b1)  // x in binary16, one power-of-two scale per token
        launch_k(k_x_to_f16, dim3(T), dim3(256), 0, st, g.x, g.H, g.K, (const int32_t*)inv,
                 at<uint16_t>(ws, L.x16), at<int8_t>(ws, L.xexp));
      if (iq2 && !b1) {  // small items (at most one per expert) and the rest
        if (large)  // 64-row items first, then the small ones, in one launch
          launch_k(k_grouped_gateup_iq2_all, dim3(g.I / kGNF, mi), dim3(kGW * 64), 0, st, g);
        else
          launch_k(k_grouped_gateup_iq2_small, dim3(g.I / kGNF, max_small_items(E, TK, T)), dim3(kGW * 64), 0, st, g);
      }
      if (q4k && !b1)
        launch_k(k_grouped_gateup_q4k, dim3((g.I + kNT - 1) / kNT, mi), dim3(256), 0, st, g);
      if (q80) {
        launch_k(k_grouped_gateup_q80, dim3(g.sh_I / kGNF, ns, g.ksplit_g), dim3(kGW * 64), 0, st, gs);
        if (g.ksplit_g > 1)
          launch_k(k_swiglu_finish, dim3((T * g.sh_I + 255) / 256), dim3(256), 0, st, g);
      } else {
        g.ksplit_g = gs.ksplit_g = 1;
      }
      if (!iq2 && !q4k && !b1)  // every item
        launch_k(k_grouped_gateup, dim3((imax + kNT - 1) / kNT, mi), dim3(256), 0, st, g);
      else if (sh && !q80)  // the shared expert's items
        launch_k(k_grouped_gateup, dim3((imax + kNT - 1) / kNT, ns), dim3(256), 0, st, gs);
    }
    if ((rc = launched()) != DS4MOE_OK) return rc;
    {
      ProfScope prof(DS4MOE_K_DOWN, st, !b1);
      const bool q2k = q2k_grouped_fast(g);
      const bool q4d = !q2k && q4k_grouped_dn(g);
      if (q2k && !b1) {  // small items and the rest
        launch_k(k_grouped_down_q2k<1>, dim3(g.H / kDNF, max_small_items(E, TK, T)), dim3(kDW * 64), 0, st, g);
        if (large) launch_k(k_grouped_down_q2k<4>, dim3(g.H / kDNF, mi), dim3(kDW * 64), 0, st, g);
      }
      if (q4d && !b1) {
        launch_k(k_grouped_down_q4k<1>, dim3(g.H / kDNF, max_small_items(E, TK, T)), dim3(kDW * 64), 0, st, g);
        if (large) launch_k(k_grouped_down_q4k<4>, dim3(g.H / kDNF, mi), dim3(kDW * 64), 0, st, g);
      }
      if (!q2k && !q4d && !b1)  // every item
        launch_k(k_grouped_down, dim3(s.hidden / kNT, mi, g.ksplit_d), dim3(256), 0, st, g);
      else if (sh)  // the shared expert's items
        launch_k(k_grouped_down, dim3(s.hidden / kNT, ns, g.ksplit_d), dim3(256), 0, st, gs);
    }
    if ((rc = launched()) != DS4MOE_OK) return rc;
    if (imx && !b1 &&
        (rc = launch_imatrix(s, *imx, x, x_dt, T, ids, wts, nullptr, 0, g.hh, g.hl, true, ws, L,
                             st)) != DS4MOE_OK)
      return rc;
    {
      ProfScope prof(DS4MOE_K_OTHER, st, !b1);
      const size_t n = (size_t)T * s.hidden;
      // the shared expert's output: y rows T*K.. (one share) or its K shares
      // in part; after the per-token matvecs k_add_shared adds it to their output
      const bool add_sh = sh && b1;
      if (!b1)
        launch_k(k_grouped_combine, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st,
                 (const float*)g.y, (const int32_t*)inv, wts, T, K, s.hidden, sh ? 1 : 0, out,
                 residual, (const float*)g.part, g.ksplit_d,
                 (((uintptr_t)out | (uintptr_t)residual) & 15) == 0 ? 1 : 0);
      if (add_sh)
        launch_k(k_add_shared, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                 (const float*)g.y, (const float*)g.part, g.ksplit_d, TK, T, s.hidden,
                 residual ? residual : out);
    }
    if ((rc = launched()) != DS4MOE_OK) return rc;
    if (perm_dbg && !b1) {
      if (hipMemcpyAsync(perm_dbg, offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToDevice, st) != hipSuccess ||
          hipMemcpyAsync(perm_dbg + E + 1, perm, sizeof(int32_t) * 2 * TK, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return DS4MOE_EDEVICE;
    }
    return DS4MOE_OK;
  }
  GenericArgs a{};
  a.x = x;
  a.x_dt = x_dt;
  a.H = s.hidden;
  a.I = ex.inter;
  a.E = s.n_expert;
  a.K = s.top_k;
  a.T = T;
  a.qt_g = ex.gate_qtype;
  a.qt_u = ex.up_qtype;
  a.qt_d = ex.down_qtype;
  a.gate = (const uint8_t*)ex.gate;
  a.up = (const uint8_t*)ex.up;
  a.down = (const uint8_t*)ex.down;
  a.grid = ex.grid;
  a.sh_I = sh ? sh->inter : 0;
  if (sh) {
    a.sh_qt_g = sh->gate_qtype;
    a.sh_qt_u = sh->up_qtype;
    a.sh_qt_d = sh->down_qtype;
    a.sh_gate = (const uint8_t*)sh->gate;
    a.sh_up = (const uint8_t*)sh->up;
    a.sh_down = (const uint8_t*)sh->down;
    a.sh_grid = sh->grid;
  }
  a.ids = ids;
  a.wts = wts;
  a.h = at<float>(ws, L.h);
  a.y = at<float>(ws, L.y);
  a.out = out;
  a.residual = residual;
  a.n_sh = sh ? T : 0;
  a.status = status;
  const int np = T * s.top_k + a.n_sh;
  const int imax = a.I > a.sh_I ? a.I : a.sh_I;
  {
    ProfScope prof(DS4MOE_K_GATEUP, st);
    launch_k(k_generic_gateup, dim3((imax + 3) / 4, np), dim3(256), 0, st, a);
  }
  ds4moe_status rc = launched();
  if (rc != DS4MOE_OK) return rc;
  {
    ProfScope prof(DS4MOE_K_DOWN, st);
    launch_k(k_generic_down, dim3((s.hidden + 3) / 4, np), dim3(256), 0, st, a);
  }
  rc = launched();
  if (rc == DS4MOE_OK && imx)  // h: fp32 [pairs][max(I, sh_I)] by pair
    rc = launch_imatrix(s, *imx, x, x_dt, T, ids, wts, a.h, imax, nullptr, nullptr, false, ws, L,
                        st);
  if (rc != DS4MOE_OK) return rc;
  size_t n = (size_t)T * s.hidden;
  {
    ProfScope prof(DS4MOE_K_OTHER, st);
    launch_k(k_generic_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  }
  return launched();
}

bool x_dtype_ok(int32_t dt) { return dt == DS4MOE_BF16 || dt == DS4MOE_F32; }

}  // namespace

DS4_EXPORT size_t ds4moe_workspace_size(const ds4moe_shape* shape, int32_t n_tok) {
  if (!shape_ok(shape) || n_tok < 0) return 0;
  return layout_for(*shape, n_tok > 0 ? n_tok : 1).total;
}

DS4_EXPORT ds4moe_status ds4moe_route(const ds4moe_shape* shape, const ds4moe_router* router,
                                      const void* x, int32_t x_dtype, int32_t n_tok,
                                      const int32_t* token_ids, int32_t* expert_ids,
                                      float* weights, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  if (!shape_ok(shape) || !router || n_tok < 0 || !expert_ids || !weights || !ws)
    return DS4MOE_EINVAL;
  if (n_tok == 0) return DS4MOE_OK;
  Layout L = layout_for(*shape, n_tok);
  if (ws_bytes < L.total) return DS4MOE_EWORKSPACE;
  if (router->tid2eid) {
    if (!token_ids || router->vocab <= 0) return DS4MOE_EINVAL;
  } else {
    if (!router->w || !router->bias || !x || !x_dtype_ok(x_dtype)) return DS4MOE_EINVAL;
    if (router->w_dtype != DS4MOE_F16 && router->w_dtype != DS4MOE_F32) return DS4MOE_EINVAL;
    if (shape->top_k > kMaxRouteK) return DS4MOE_EUNSUPPORTED;
  }
  return do_route(*shape, *router, x, x_dtype, nullptr, nullptr, 0.0f, nullptr, n_tok, token_ids,
                  expert_ids, weights, ws, L, stream);
}

DS4_EXPORT ds4moe_status ds4moe_permute(const ds4moe_shape* shape, const int32_t* expert_ids,
                                        int32_t n_tok, int32_t* counts, int32_t* offsets,
                                        int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (!shape_ok(shape) || !expert_ids || !counts || !offsets || !perm || !inv || !ws || n_tok < 0)
    return DS4MOE_EINVAL;
  if ((int64_t)n_tok * shape->top_k > 32768) return DS4MOE_EUNSUPPORTED;
  if (n_tok == 0) return DS4MOE_OK;
  Layout L = layout_for(*shape, n_tok);
  if (ws_bytes < L.total) return DS4MOE_EWORKSPACE;
  ProfScope prof(DS4MOE_K_PERMUTE, stream);
  return launch_permute(expert_ids, n_tok * shape->top_k, shape->n_expert, counts, offsets, perm,
                        inv, at<uint32_t>(ws, L.status), stream);
}

DS4_EXPORT ds4moe_status ds4moe_expert_ffn(const ds4moe_shape* shape,
                                           const ds4moe_experts* routed,
                                           const ds4moe_experts* shared, const void* x,
                                           int32_t x_dtype, int32_t n_tok,
                                           const int32_t* expert_ids, const float* weights,
                                           float* out, int32_t* perm_dbg, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  if (!shape_ok(shape) || !experts_ok(routed, shape->hidden) || !x || !x_dtype_ok(x_dtype) ||
      !expert_ids || !weights || !out || !ws || n_tok < 0)
    return DS4MOE_EINVAL;
  if (routed->inter != shape->inter) return DS4MOE_EINVAL;
  if (shared && (!experts_ok(shared, shape->hidden) || shared->inter > shape->inter))
    return DS4MOE_EINVAL;
  if (n_tok == 0) return DS4MOE_OK;
  Layout L = layout_for(*shape, n_tok);
  if (ws_bytes < L.total) return DS4MOE_EWORKSPACE;
  if ((int64_t)n_tok * shape->top_k > 32768) return DS4MOE_EUNSUPPORTED;
  return do_ffn(*shape, *routed, shared, x, x_dtype, n_tok, expert_ids, weights, out, nullptr,
                perm_dbg, ws, L, stream);
}

DS4_EXPORT ds4moe_status ds4moe_expert_ffn_imatrix(const ds4moe_shape* shape,
                                                   const ds4moe_experts* routed,
                                                   const ds4moe_experts* shared, const void* x,
                                                   int32_t x_dtype, int32_t n_tok,
                                                   const int32_t* expert_ids, const float* weights,
                                                   float* out, float* imx_gateup, float* imx_down,
                                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!shape_ok(shape) || !experts_ok(routed, shape->hidden) || !x || !x_dtype_ok(x_dtype) ||
      !expert_ids || !weights || !out || !imx_gateup || !imx_down || !ws || n_tok < 0)
    return DS4MOE_EINVAL;
  if (routed->inter != shape->inter) return DS4MOE_EINVAL;
  if (shared && (!experts_ok(shared, shape->hidden) || shared->inter > shape->inter))
    return DS4MOE_EINVAL;
  if (n_tok == 0) return DS4MOE_OK;
  Layout L = layout_for(*shape, n_tok);
  if (ws_bytes < L.total) return DS4MOE_EWORKSPACE;
  if ((int64_t)n_tok * shape->top_k > 32768) return DS4MOE_EUNSUPPORTED;
  const ImxOut imx{imx_gateup, imx_down};
  return do_ffn(*shape, *routed, shared, x, x_dtype, n_tok, expert_ids, weights, out, nullptr,
                nullptr, ws, L, stream, &imx);
}

namespace {

// Argument checks of ds4moe_layer (all but the workspace).
ds4moe_status layer_args(const ds4moe_shape* shape, const ds4moe_layer_desc* desc, const void* x,
                         int32_t x_dtype, float* residual, float* out, const int32_t* token_ids,
                         int32_t n_tok) {
  if (!shape_ok(shape) || !desc || !experts_ok(&desc->routed, shape->hidden) || n_tok < 0)
    return DS4MOE_EINVAL;
  if (desc->routed.inter != shape->inter) return DS4MOE_EINVAL;
  const ds4moe_experts* sh = desc->shared;
  if (sh && (!experts_ok(sh, shape->hidden) || sh->inter > shape->inter)) return DS4MOE_EINVAL;
  const ds4moe_router& r = desc->router;
  if (r.tid2eid) {
    if (!token_ids || r.vocab <= 0) return DS4MOE_EINVAL;
  } else if (!r.w || !r.bias || (r.w_dtype != DS4MOE_F16 && r.w_dtype != DS4MOE_F32)) {
    return DS4MOE_EINVAL;
  } else if (shape->top_k > kMaxRouteK) {
    return DS4MOE_EUNSUPPORTED;
  }
  if (desc->norm_w) {
    if (!residual) return DS4MOE_EINVAL;
  } else {
    if (!x || !x_dtype_ok(x_dtype) || !out) return DS4MOE_EINVAL;
  }
  if ((int64_t)n_tok * shape->top_k > 32768) return DS4MOE_EUNSUPPORTED;
  return DS4MOE_OK;
}

// The layer on a workspace of layout L (arguments checked, n_tok > 0).
ds4moe_status layer_run(const ds4moe_shape* shape, const ds4moe_layer_desc* desc, const void* x,
                        int32_t x_dtype, float* residual, float* out, const int32_t* token_ids,
                        int32_t n_tok, int32_t* ids_dbg, float* w_dbg, uint16_t* xn_dbg, void* ws,
                        const Layout& L, hipStream_t stream) {
  const ds4moe_experts* sh = desc->shared;
  const ds4moe_router& r = desc->router;
  const bool norm = desc->norm_w != nullptr;
  int32_t* ids = at<int32_t>(ws, L.ids);
  float* wts = at<float>(ws, L.wts);
  uint16_t* xn = at<uint16_t>(ws, L.xn);
  ds4moe_status rc;
  // hash-routed layers with an RMSNorm: one launch normalises and routes
  const bool norm_hash = norm && r.tid2eid;
  if (norm_hash) {
    ProfScope prof(DS4MOE_K_OTHER, stream);
    const HashArgs hs{token_ids, r.tid2eid, r.vocab, shape->n_expert, shape->top_k,
                      shape->routed_scale, ids, wts, at<uint32_t>(ws, L.status)};
    launch_k(k_rmsnorm_bf16, dim3(n_tok), dim3(256), 0, stream, residual, desc->norm_w,
                       desc->norm_eps, shape->hidden, xn, hs);
    if ((rc = launched()) != DS4MOE_OK) return rc;
  }
  const void* fx = norm ? (const void*)xn : x;
  int32_t fdt = norm ? (int32_t)DS4MOE_BF16 : x_dtype;
  // few-token path with a learned router, up to kFuseSelMaxTokens tokens: the
  // top-6 selection of each token runs inside the gate/up kernel (one kernel
  // boundary fewer; with more tokens every round of gate/up blocks would pay
  // the selection's latency, which costs what the boundary saves)
  const bool fuse = !r.tid2eid && n_tok <= kFuseSelMaxTokens &&
                    fast_b1(*shape, desc->routed, fx, fdt, n_tok) &&
                    (!sh || grouped_eligible(*shape, desc->routed, sh, fx, fdt, n_tok));
  // selection kernel before the few-token matvecs: it also lists the
  // distinct experts for the IQ2_XXS gate/up that reads each once
  const bool few_items = !fuse && !r.tid2eid && n_tok >= kFewMinT &&
                         n_tok * shape->top_k <= kSelItemsMax && n_tok <= 16 &&
                         desc->routed.gate_qtype == DS4MOE_IQ2_XXS &&
                         fast_b1(*shape, desc->routed, fx, fdt, n_tok, true) &&
                         (!sh || grouped_eligible(*shape, desc->routed, sh, fx, fdt, n_tok));
  // the shared expert's gate/up runs in the scoring launch when it goes by
  // matvecs (with an RMSNorm, per-token kernels whose blocks normalise the
  // input themselves)
  const bool sh_union =
      sh && !r.tid2eid &&
      shared_by_matvecs(*shape, desc->routed, sh, fx, fdt, n_tok, few_items && !fuse) &&
      (!norm || (n_tok <= kSharedB1MaxTokens &&
                 route_vec(*shape, r, x, x_dtype, residual, desc->norm_w, xn)));
  const SharedB1Args shu =
      sh_union ? shared_args(*shape, *sh, fx, n_tok, out, residual, ws, L) : SharedB1Args{};
  if (!norm_hash) {
    rc = do_route(*shape, r, x, x_dtype, norm ? residual : nullptr, norm ? desc->norm_w : nullptr,
                  desc->norm_eps, norm ? xn : nullptr, n_tok, token_ids, ids, wts, ws, L, stream,
                  !fuse, few_items, sh_union ? &shu : nullptr);
    if (rc != DS4MOE_OK) return rc;
  }
  // the fused selection reads the router input fx (the normalised row when
  // norm: the scoring wrote it to the workspace) for exact recomputations
  rc = do_ffn(*shape, desc->routed, sh, fx, fdt, n_tok, ids, wts, norm ? nullptr : out,
              norm ? residual : nullptr, nullptr, ws, L, stream, nullptr,
              fuse ? at<float4>(ws, L.kbuf) : nullptr, fuse ? &r : nullptr, few_items, sh_union);
  if (rc != DS4MOE_OK) return rc;
  if (ids_dbg &&
      hipMemcpyAsync(ids_dbg, ids, sizeof(int32_t) * n_tok * shape->top_k, hipMemcpyDeviceToDevice,
                     stream) != hipSuccess)
    return DS4MOE_EDEVICE;
  if (w_dbg && hipMemcpyAsync(w_dbg, wts, sizeof(float) * n_tok * shape->top_k,
                              hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return DS4MOE_EDEVICE;
  if (xn_dbg && norm &&
      hipMemcpyAsync(xn_dbg, xn, sizeof(uint16_t) * (size_t)n_tok * shape->hidden,
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return DS4MOE_EDEVICE;
  return DS4MOE_OK;
}

}  // namespace

DS4_EXPORT ds4moe_status ds4moe_layer(const ds4moe_shape* shape, const ds4moe_layer_desc* desc,
                                      const void* x, int32_t x_dtype, float* residual, float* out,
                                      const int32_t* token_ids, int32_t n_tok, int32_t* ids_dbg,
                                      float* w_dbg, uint16_t* xn_dbg, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  if (!ws) return DS4MOE_EINVAL;
  ds4moe_status rc = layer_args(shape, desc, x, x_dtype, residual, out, token_ids, n_tok);
  if (rc != DS4MOE_OK || n_tok == 0) return rc;
  const Layout L = layout_for(*shape, n_tok);
  if (ws_bytes < L.total) return DS4MOE_EWORKSPACE;
  return layer_run(shape, desc, x, x_dtype, residual, out, token_ids, n_tok, ids_dbg, w_dbg,
                   xn_dbg, ws, L, stream);
}

// ---- allocation-free layer call -------------------------------------------------
// The workspace of ds4moe_layer_noalloc: one static device array per GPU,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to kernels.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kScratchMaxDevices] = {};

// The current device's address of `scratch` (nullptr if it cannot be had).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_dev[dev] = p;
  }
  return g_scratch_dev[dev];
}

// Clears the status region at the start of the scratch workspace (a kernel,
// not a memset, so that the call can be captured into a graph).
__global__ void k_scratch_clear(uint32_t* status) { status[threadIdx.x] = 0u; }

__global__ void k_scratch_faults(const uint32_t* status, uint32_t* faults) { *faults = *status; }

}  // namespace

DS4_EXPORT ds4moe_status ds4moe_layer_noalloc(const ds4moe_shape* shape,
                                              const ds4moe_layer_desc* desc, const void* x,
                                              int32_t x_dtype, float* residual, float* out,
                                              const int32_t* token_ids, int32_t n_tok,
                                              int32_t* ids_dbg, float* w_dbg, uint16_t* xn_dbg,
                                              uint32_t* faults, hipStream_t stream) {
  ds4moe_status rc = layer_args(shape, desc, x, x_dtype, residual, out, token_ids, n_tok);
  if (rc != DS4MOE_OK || n_tok == 0) return rc;
  const Layout L = layout_for(*shape, n_tok);
  if (L.total > kScratchBytes) return DS4MOE_EWORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return DS4MOE_EDEVICE;
  {
    ProfScope prof(DS4MOE_K_OTHER, stream);
    launch_k(k_scratch_clear, dim3(1), dim3(64), 0, stream, static_cast<uint32_t*>(ws));
  }
  if ((rc = launched()) != DS4MOE_OK) return rc;
  rc = layer_run(shape, desc, x, x_dtype, residual, out, token_ids, n_tok, ids_dbg, w_dbg, xn_dbg,
                 ws, L, stream);
  if (rc != DS4MOE_OK || !faults) return rc;
  ProfScope prof(DS4MOE_K_OTHER, stream);
  launch_k(k_scratch_faults, dim3(1), dim3(1), 0, stream, static_cast<const uint32_t*>(ws), faults);
  return launched();
}

namespace {

// Streaming-read probe: workgroup b reads the b-th contiguous chunk of the
// buffer, each thread keeping eight 16-byte loads in flight; the data are
// folded into a checksum so that no load can be dropped.
constexpr int kProbeGroups = 4096, kProbeThreads = 256, kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const uint4* __restrict__ src,
                                                             size_t n16, uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = (size_t)blockIdx.x * per, e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  for (size_t i = b + threadIdx.x; i < e; i += (size_t)kProbeThreads * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) {
      const size_t j = i + (size_t)u * kProbeThreads;
      v[u] = j < e ? src[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one writer per workgroup, in a fixed slot: the checksum is the same on
  // every run (the XOR of the workgroups' values)
  acc = __reduce_xor_sync(0xFFFFFFFFFFFFFFFFull, acc);
  __shared__ uint32_t wv[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) wv[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(sink, wv[0] ^ wv[1] ^ wv[2] ^ wv[3]);
}

}  // namespace

DS4_EXPORT ds4moe_status ds4moe_read_probe(const void* src, size_t bytes, uint32_t* sink,
                                           hipStream_t stream) {
  if (!src || !sink || ((uintptr_t)src & 15) || (bytes & 15)) return DS4MOE_EINVAL;
  if (bytes == 0) return DS4MOE_OK;
  launch_k(k_read_probe, dim3(kProbeGroups), dim3(kProbeThreads), 0, stream,
           static_cast<const uint4*>(src), bytes / 16, sink);
  return launched();
}

DS4_EXPORT ds4moe_status ds4moe_profile_events(int32_t cls, hipEvent_t begin, hipEvent_t end) {
  if (cls < 0 || cls >= DS4MOE_K_CLASSES) return DS4MOE_EINVAL;
  g_prof[cls][0] = begin;
  g_prof[cls][1] = end;
  return DS4MOE_OK;
}

// ---------------------------------------------------------------------------
// Block encoders (encode.hip)
// ---------------------------------------------------------------------------
DS4_EXPORT size_t ds4moe_iq2_map_bytes(void) { return kIq2MapBytes; }

DS4_EXPORT ds4moe_status ds4moe_iq2_map_build(const uint8_t* grid, void* map, void* ws,
                                              size_t ws_bytes, hipStream_t stream) {
  if (!grid || !map || !ws || ws_bytes < 256 || ((uintptr_t)grid & 7) || ((uintptr_t)map & 1))
    return DS4MOE_EINVAL;
  ProfScope prof(DS4MOE_K_OTHER, stream);
  launch_k(k_iq2_map, dim3((kIq2Keys + 3) / 4), dim3(kEncThreads), 0, stream, grid,
           static_cast<uint8_t*>(map), at<uint32_t>(ws, 0));
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_EDEVICE;
}

DS4_EXPORT ds4moe_status ds4moe_quantize(int32_t qtype, const float* src, int64_t n_mats,
                                         int64_t rows, int64_t cols, const float* importance,
                                         int64_t imp_stride, const uint8_t* grid,
                                         const void* iq2_map, void* dst, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  if (!qtype_ok(qtype) || !src || !dst || !ws ||
      ws_bytes < 256 || n_mats < 0 || rows < 0 || cols < 0 || cols % 256 || imp_stride < 0 ||
      imp_stride % 4 || ((uintptr_t)src & 15) || ((uintptr_t)importance & 15))
    return DS4MOE_EINVAL;
  if (qtype == DS4MOE_IQ2_XXS &&
      (!importance || !grid || !iq2_map || ((uintptr_t)grid & 7) || ((uintptr_t)iq2_map & 1) ||
       ((uintptr_t)dst & 1)))
    return DS4MOE_EINVAL;
  if (qtype == DS4MOE_Q2_K && ((uintptr_t)dst & 3)) return DS4MOE_EINVAL;
  if (qtype == DS4MOE_Q4_K && ((uintptr_t)dst & 15)) return DS4MOE_EINVAL;
  if (qtype == DS4MOE_Q8_0 && ((uintptr_t)dst & 1)) return DS4MOE_EINVAL;
  // blocks of 256 values (Q8_0: of 32)
  const int64_t n_blocks = n_mats * rows * (cols / (qtype == DS4MOE_Q8_0 ? 32 : 256));
  if (n_blocks == 0) return DS4MOE_OK;
  EncArgs a;
  a.src = src;
  a.imp = importance;
  a.grid = grid;
  a.map = static_cast<const uint8_t*>(iq2_map);
  a.dst = static_cast<uint8_t*>(dst);
  a.status = at<uint32_t>(ws, 0);
  a.n_blocks = n_blocks;
  a.bpr = cols / 256;
  a.rows = rows;
  a.imp_stride = imp_stride;
  ProfScope prof(DS4MOE_K_OTHER, stream);
  const int per = qtype == DS4MOE_Q2_K ? kEncThreads / 16
                  : qtype == DS4MOE_Q8_0 ? kEncThreads
                                         : kEncThreads / 8;
  const int64_t wgs = (n_blocks + per - 1) / per;
  if (wgs > 0x7FFFFFFF) return DS4MOE_EUNSUPPORTED;
  if (qtype == DS4MOE_Q2_K)
    launch_k(k_encode_q2k, dim3((uint32_t)wgs), dim3(kEncThreads), 0, stream, a);
  else if (qtype == DS4MOE_Q4_K)
    launch_k(k_encode_q4k, dim3((uint32_t)wgs), dim3(kEncThreads), 0, stream, a);
  else if (qtype == DS4MOE_Q8_0)
    launch_k(k_encode_q80, dim3((uint32_t)wgs), dim3(kEncThreads), 0, stream, a);
  else
    launch_k(k_encode_iq2, dim3((uint32_t)wgs), dim3(kEncThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_EDEVICE;
}

DS4_EXPORT ds4moe_status ds4moe_column_energy(const float* src, int64_t n_mats, int64_t rows,
                                              int64_t cols, float* out, hipStream_t stream) {
  if (!src || !out || n_mats < 0 || rows < 0 || cols < 0) return DS4MOE_EINVAL;
  const int64_t n = n_mats * cols;
  if (n == 0) return DS4MOE_OK;
  const int64_t wgs = (n + kEncThreads - 1) / kEncThreads;
  if (wgs > 0x7FFFFFFF) return DS4MOE_EUNSUPPORTED;
  ProfScope prof(DS4MOE_K_OTHER, stream);
  launch_k(k_column_energy, dim3((uint32_t)wgs), dim3(kEncThreads), 0, stream, src, n_mats, rows,
           cols, out);
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_EDEVICE;
}

DS4_EXPORT ds4moe_status ds4moe_check(void* ws, hipStream_t stream, uint32_t* faults) {
  if (!ws) return DS4MOE_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return DS4MOE_EDEVICE;
  uint32_t v = 0, zero = 0;
  if (hipMemcpy(&v, ws, 4, hipMemcpyDeviceToHost) != hipSuccess) return DS4MOE_EDEVICE;
  if (v && hipMemcpy(ws, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return DS4MOE_EDEVICE;
  if (faults) *faults = v;
  return v ? DS4MOE_EDATA : DS4MOE_OK;
}

DS4_EXPORT const char* ds4moe_status_string(ds4moe_status s) {
  switch (s) {
    case DS4MOE_OK: return "ok";
    case DS4MOE_EINVAL: return "invalid argument";
    case DS4MOE_EUNSUPPORTED: return "unsupported shape or type";
    case DS4MOE_EWORKSPACE: return "workspace too small";
    case DS4MOE_EDEVICE: return "HIP call failed";
    case DS4MOE_EDATA: return "device-detected data fault";
  }
  return "unknown status";
}
