/*
 * ds4moe.h -- C ABI of libds4moe: the DeepSeek-V4-Flash routed-expert MoE
 * FFN on block-quantised 2-bit weights, for AMD MI355X (gfx950).
 *
 * The method (pages: FLOW = qiita.com/sukimaengineer/items/cd76fec76d49a098abed,
 * section "MoE FFN 部の中身: router -> top-6 -> expert -> 加重和" and the
 * config table; DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec,
 * sections 3 "Q2_K" and 4 "IQ2_XXS"):
 *   logits   z = x . W_r^T                 (router, f16 weights)
 *   scores   s = sqrtsoftplus(z) = sqrt(ln(1 + e^z))
 *   select   the top_k of key = s + bias   (bias for selection only)
 *   gates    g = routed_scale * s_sel / sum(s_sel)
 *   experts  E(x) = W_down (SiLU(W_gate x) * W_up x)
 *   output   y = shared(x) + sum_k g_k E_k(x)
 * with the first layers routed by a static token-id table instead
 * (FLOW: hash routing in layers 0-2, no router there).
 *
 * Conventions for every entry point:
 *  - Data pointers are DEVICE pointers (hipMalloc'd or equivalent) unless
 *    stated; the caller owns all memory.  Calls only enqueue work on
 *    `stream` and return without waiting; nothing is allocated.
 *  - Arguments are checked on the host before anything is launched; a
 *    negative status means nothing was enqueued.
 *  - Faults in the data that only the device can see (an expert id out of
 *    range in caller-given routing, a bad hash-table row, a token id out of
 *    range) set bits of a
 *    status word in the workspace; ds4moe_check() reports them.  Such data
 *    never causes an out-of-bounds access: offending ids are replaced by
 *    valid ones before use.
 *  - The workspace `ws` (ws_bytes >= ds4moe_workspace_size()) must be
 *    zero-filled once before its first use; every call leaves its internal
 *    counters at zero again.  Calls sharing one workspace must be ordered
 *    on one stream.
 *  - No exceptions cross the ABI.  NaN or Inf in activations propagate.
 */
#ifndef DS4MOE_H
#define DS4MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DS4MOE_OK = 0,
  DS4MOE_EINVAL = -1,      /* bad argument (null, size, alignment, dtype) */
  DS4MOE_EUNSUPPORTED = -2,/* valid but not implemented for this shape/type */
  DS4MOE_EWORKSPACE = -3,  /* workspace smaller than ds4moe_workspace_size */
  DS4MOE_EDEVICE = -4,     /* a HIP call failed */
  DS4MOE_EDATA = -5        /* device-detected data fault (ds4moe_check) */
} ds4moe_status;

typedef enum { DS4MOE_F32 = 0, DS4MOE_F16 = 1, DS4MOE_BF16 = 2 } ds4moe_dtype;

/* Block formats (DS4C2 sections 3 and 4; FLOW quantisation table):
 *  Q2_K      84 B / 256 values: 16 B scale|min nibbles, 64 B 2-bit codes,
 *            fp16 d, fp16 dmin;  y = d*sc*q - dmin*m
 *  IQ2_XXS   66 B / 256 values: fp16 d, 8 groups of (4 grid-index bytes,
 *            u32 of 4x7 sign bits + 4-bit scale s); y = d*(2s+1)/8*grid*sign
 *  Q8_0      34 B / 32 values: fp16 d, 32 int8; y = d*c
 *  Q4_K      144 B / 256 values (size from the DS4C2 type table; layout of
 *            the k-quant family): fp16 d, fp16 dmin, 12 B of 6-bit scale and
 *            min per 32-value sub-block, 128 B of 4-bit codes (byte 32c+l:
 *            values 64c+l low nibble, 64c+32+l high); y = d*sc*q - dmin*m    */
typedef enum { DS4MOE_Q2_K = 0, DS4MOE_IQ2_XXS = 1, DS4MOE_Q8_0 = 2, DS4MOE_Q4_K = 3 } ds4moe_qtype;

/* Layer shape.  hidden must be a multiple of 256 and inter of 32 (blocks
 * tile the row-major flattening of each matrix, so a block may span rows);
 * top_k <= n_expert <= 256, top_k <= 64 (learned routers: top_k <= 16). */
typedef struct {
  int32_t hidden;       /* H (4096)                                    */
  int32_t inter;        /* routed expert intermediate size I (2048)    */
  int32_t n_expert;     /* E (256)                                     */
  int32_t top_k;        /* K (6)                                       */
  float routed_scale;   /* routed_scaling_factor (1.5)                 */
} ds4moe_shape;

/* A stacked set of SwiGLU experts.  gate and up are [n][inter][hidden],
 * down is [n][hidden][inter]; each matrix is the row-major flattening cut
 * into consecutive blocks of its qtype (all experts of a layer in one
 * tensor, expert e starting at e * rows * cols / values_per_block blocks).
 * Pointers must be 4-byte aligned.  `grid` (IQ2_XXS only) is 256 x 8 bytes
 * of grid values (each < 128). */
typedef struct {
  int32_t gate_qtype, up_qtype, down_qtype;
  const void* gate;
  const void* up;
  const void* down;
  int32_t inter;          /* intermediate size of these experts */
  const uint8_t* grid;    /* device, required if any qtype is IQ2_XXS */
} ds4moe_experts;

/* Router of one layer.  Either a learned router (w != NULL: [n_expert][hidden]
 * of w_dtype F16 or F32, plus fp32 bias[n_expert] used only for selection),
 * or a hash layer (tid2eid != NULL: int32 [vocab][top_k], expert ids per token
 * id, equal gates routed_scale / top_k). */
typedef struct {
  const void* w;
  int32_t w_dtype;
  const float* bias;
  const int32_t* tid2eid;
  int32_t vocab;
} ds4moe_router;

/* One MoE layer for ds4moe_layer(). */
typedef struct {
  ds4moe_router router;
  ds4moe_experts routed;           /* n = n_expert */
  const ds4moe_experts* shared;    /* host pointer to a descriptor of one
                                      always-on expert, or NULL */
  const float* norm_w;             /* fp32 [hidden] RMSNorm weight, or NULL */
  float norm_eps;
} ds4moe_layer_desc;

/* Bytes of workspace needed for n_tok tokens of this shape (0 on bad shape). */
size_t ds4moe_workspace_size(const ds4moe_shape* shape, int32_t n_tok);

/*
 * Routing (FLOW "MoE FFN" section): for each of n_tok tokens write the top_k
 * expert ids (int32 [n_tok][top_k], slots ordered by key descending, ties to
 * the lower expert index) and gate weights (fp32 [n_tok][top_k], summing to
 * routed_scale).  x: [n_tok][hidden] of x_dtype (BF16 or F32).
 * Learned router: logits are the exact dot products rounded once to fp32,
 * scores are sqrtsoftplus rounded to fp32 (correctly rounded), keys are fp32
 * score + bias.  The device accumulates logits in fp64 and evaluates scores
 * in fp64, each with an error bound; where the bounds leave the selection
 * open, the keys that could still be selected are recomputed exactly
 * (integer-limb logit, double-double score with a 2^-90 error bound).  Only a
 * score within 2^-90 (relative) of a binary32 rounding point, where even the
 * double-double evaluation cannot decide, would set DS4MOE_FAULT_UNCERTIFIED
 * (the selection then uses the nearer rounding); none is known.
 * Hash layer: token_ids (int32 [n_tok], required) index tid2eid; token ids
 * outside [0, vocab) or table rows with ids out of range or repeated set a
 * fault bit and route that token to experts 0..top_k-1.
 */
ds4moe_status ds4moe_route(const ds4moe_shape* shape, const ds4moe_router* router, const void* x,
                           int32_t x_dtype, int32_t n_tok, const int32_t* token_ids,
                           int32_t* expert_ids, float* weights, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * Token -> expert permutation: pair p = t*top_k + k is ordered by
 * (expert, t, k).  counts int32 [n_expert], offsets int32 [n_expert+1]
 * (exclusive prefix sum), perm int32 [n_tok*top_k] (pair at each sorted
 * position), inv int32 [n_tok*top_k] (position of each pair).  Ids outside
 * [0, n_expert) set DS4MOE_FAULT_BAD_ID and are counted as expert 0.
 * n_tok * top_k <= 32768.
 */
ds4moe_status ds4moe_permute(const ds4moe_shape* shape, const int32_t* expert_ids, int32_t n_tok,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Expert FFN and weighted combine (FLOW "MoE FFN" section):
 *   out[t] = sum_k weights[t][k] * E_{expert_ids[t][k]}(x[t])  + shared(x[t])
 * x: [n_tok][hidden] BF16 or F32; out: fp32 [n_tok][hidden].  `shared` may
 * be NULL.  Accumulation is fp32: dot products of exact products (decode
 * paths with the V4-Flash shape and formats: up to 8 tokens with IQ2_XXS
 * gate/up and Q2_K down (10 in ds4moe_layer calls, whose selection lists
 * the distinct experts), up to 13 with Q4_K gate/up or down) or MFMAs on
 * exact binary16/bf16 operands
 * (grouped path, more tokens; gate/up IQ2_XXS, Q8_0 or both Q4_K, down Q2_K,
 * Q8_0 or Q4_K); other combinations run on scalar kernels.  The permutation
 * used for n_tok > 1 may be captured: perm_dbg (nullable) receives
 * offsets[n_expert+1], perm[n_tok*top_k], inv[n_tok*top_k] (int32).
 */
ds4moe_status ds4moe_expert_ffn(const ds4moe_shape* shape, const ds4moe_experts* routed,
                                const ds4moe_experts* shared, const void* x, int32_t x_dtype,
                                int32_t n_tok, const int32_t* expert_ids, const float* weights,
                                float* out, int32_t* perm_dbg, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * ds4moe_expert_ffn, plus the importance statistics of the routed experts'
 * inputs ("imatrix", DS4C2 = qiita.com/yoshiyakato/items/4678be0e7860ddb444ec,
 * sections 5 and 7: activation statistics per input column, one entry of
 * n_expert * n_columns values per expert tensor).  For every pair (t, k)
 * with e = expert_ids[t][k]:
 *   imx_gateup[e][c] += x[t][c]^2                   c < hidden
 *       (the gate and up input; x is the FFN-normalised activation)
 *   imx_down[e][i]   += (weights[t][k] * h[t][k][i])^2   i < inter
 *       (the down input: the pair's SwiGLU row after its routing weight)
 * imx_gateup: fp32 [n_expert][hidden], imx_down: fp32 [n_expert][inter],
 * device, caller-owned, accumulated into (zero them before a calibration
 * run); each call adds its own sums (fp64 in a fixed order inside the call,
 * one fp32 rounding per element per call): repeated calls on the same inputs
 * add bit-identical amounts.  h is
 * the SwiGLU row the FFN computed (fp32, or binary16 high + low parts on the
 * grouped path, relative error < 2^-21).  The shared expert has no entry.
 * Same arguments, errors and workspace as ds4moe_expert_ffn (no perm_dbg);
 * both statistics pointers are required.
 */
ds4moe_status ds4moe_expert_ffn_imatrix(const ds4moe_shape* shape, const ds4moe_experts* routed,
                                        const ds4moe_experts* shared, const void* x,
                                        int32_t x_dtype, int32_t n_tok, const int32_t* expert_ids,
                                        const float* weights, float* out, float* imx_gateup,
                                        float* imx_down, void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/*
 * A whole MoE layer.  If desc->norm_w is set: xn = RMSNorm(residual)
 * (fp32 [n_tok][hidden] in, bf16 out; mean of squares in fp64), the layer
 * runs on xn and residual += y (fp32), `x` is ignored and `out` may be NULL.
 * Otherwise it runs on x and writes y to out (residual ignored).
 * token_ids are required for hash layers.  Debug captures (nullable): ids_dbg
 * int32 [n_tok][top_k], w_dbg fp32 [n_tok][top_k], xn_dbg bf16 bits
 * [n_tok][hidden].
 */
ds4moe_status ds4moe_layer(const ds4moe_shape* shape, const ds4moe_layer_desc* desc, const void* x,
                           int32_t x_dtype, float* residual, float* out,
                           const int32_t* token_ids, int32_t n_tok, int32_t* ids_dbg, float* w_dbg,
                           uint16_t* xn_dbg, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ds4moe_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results as ds4moe_layer, without the
 * workspace arguments.  Its workspace is a static device array of 8 MiB per
 * GPU (part of the library's device code, present on every GPU the library
 * runs on until the process ends); the call itself allocates nothing.  n_tok must satisfy
 * ds4moe_workspace_size(shape, n_tok) <= 8 MiB (up to 17 tokens with the
 * V4-Flash shape: hidden 4096, inter 2048, 256 experts, top-6), otherwise
 * DS4MOE_EWORKSPACE is returned before anything is enqueued.  faults
 * (device, nullable): one uint32 that receives this call's fault bits (the
 * bits ds4moe_check reports; 0 when clean) when the call's work completes.
 * Every call on a GPU uses that GPU's one array (its status word is cleared
 * at the start of each call): calls that overlap on one GPU (two streams or
 * host threads without ordering) race and must be ordered on one stream.
 */
ds4moe_status ds4moe_layer_noalloc(const ds4moe_shape* shape, const ds4moe_layer_desc* desc,
                                   const void* x, int32_t x_dtype, float* residual, float* out,
                                   const int32_t* token_ids, int32_t n_tok, int32_t* ids_dbg,
                                   float* w_dbg, uint16_t* xn_dbg, uint32_t* faults,
                                   hipStream_t stream);

/* Status-word bits reported by ds4moe_check(). */
#define DS4MOE_FAULT_BAD_ID 0x1u       /* caller-given expert id out of range   */
#define DS4MOE_FAULT_BAD_TOKEN 0x2u    /* token id outside [0, vocab)           */
#define DS4MOE_FAULT_BAD_TABLE 0x4u    /* tid2eid row out of range / repeated   */
#define DS4MOE_FAULT_UNCERTIFIED 0x8u  /* a score undecidable even in double-
                                          double arithmetic (see route)       */
#define DS4MOE_FAULT_F16_RANGE 0x10u   /* reserved: not raised (binary16
                                          operands are scaled by powers of two) */
#define DS4MOE_FAULT_BAD_INPUT 0x20u   /* encoder: non-finite value, negative or
                                          non-finite importance, grid value not
                                          8, 25 or 43                            */

/* Kernel classes for ds4moe_profile_events(). */
#define DS4MOE_K_ROUTE 0     /* router scoring + selection, or hash lookup  */
#define DS4MOE_K_GATEUP 1    /* gate/up matvec + SwiGLU (any path)          */
#define DS4MOE_K_DOWN 2      /* down matvec + combine (any path)            */
#define DS4MOE_K_PERMUTE 3   /* token -> expert permutation                 */
#define DS4MOE_K_OTHER 4     /* RMSNorm, combine, quantisation helpers      */
#define DS4MOE_K_CLASSES 5

/*
 * Profiling hook (measurement only, not part of the method).  After this
 * call every launch of kernel class `cls` is bracketed by
 * hipEventRecord(begin) and hipEventRecord(end) on the stream it is launched
 * on; pass NULL events to stop.  The events are caller-owned HIP events.
 * Process-wide setting, not thread-safe: set it between calls from one host
 * thread.  Returns DS4MOE_EINVAL for an unknown class.
 */
ds4moe_status ds4moe_profile_events(int32_t cls, hipEvent_t begin, hipEvent_t end);

/*
 * Streaming-read probe (measurement only, not part of the method): reads
 * `bytes` bytes at `src` (device, 16-byte aligned, bytes a multiple of 16)
 * once with 16-byte vector loads, as a plain streaming kernel that does no
 * other work (4096 workgroups of 256 threads, each reading one contiguous
 * chunk, eight loads in flight per thread), and writes a checksum of the
 * data to *sink (device).  Timing it gives the read bandwidth the memory
 * system delivers to a kernel on this device, against which the expert
 * kernels' bandwidth is quoted.  Asynchronous on `stream`.
 */
ds4moe_status ds4moe_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Block encoders: fp32 matrices -> Q2_K / IQ2_XXS blocks               */
/* ------------------------------------------------------------------ */
/*
 * Defined by DS4C2 (qiita.com/yoshiyakato/items/4678be0e7860ddb444ec)
 * sec. 3 (Q2_K: a scale and a min per 16 values, 2-bit codes; with an
 * importance vector the weighted variant, whose per-column importance
 * weighs the quantisation error), sec. 4 (IQ2_XXS: requires importance;
 * tuples off the 256-entry grid are searched in a two-shell neighbour list),
 * sec. 5, 7, 8 (importance = sum of squared activations per column, one
 * vector per expert; fallback = column energy of the weights).  The pages
 * print no search procedure: the library carries out a fixed one (least-
 * squares refits for Q2_K, 16 candidate group scales for IQ2_XXS) with every
 * decision in binary32 in a stated order; the exact steps are written at the
 * kernels (encode.hip).  Outputs are deterministic: the same input gives the
 * same bytes on every call and launch configuration.
 */

/* Bytes of an IQ2_XXS neighbour map: uint16 count[6561], then uint8
 * idx[6561][256] (6561 = 3^8 tuples of the levels 8, 25, 43). */
size_t ds4moe_iq2_map_bytes(void);

/*
 * Builds the neighbour map of an IQ2_XXS grid.  grid: device, 256 x 8 bytes,
 * 8-byte aligned, every byte 8, 25 or 43.  map: device, ds4moe_iq2_map_bytes()
 * bytes, caller-owned.  For the tuple of levels with key sum_k level_k 3^k
 * the list holds the lowest grid index equal to it, or, off the grid, every
 * index whose squared level distance is at most the second-smallest distance
 * over the grid, ascending.  ws: a zero-filled workspace of >= 256 bytes (its
 * status word; any workspace of this library serves); a grid byte outside
 * {8, 25, 43} sets DS4MOE_FAULT_BAD_INPUT.  Asynchronous on `stream`.
 */
ds4moe_status ds4moe_iq2_map_build(const uint8_t* grid, void* map, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * Encodes n_mats row-major fp32 matrices [rows][cols] (stacked, device,
 * 16-byte aligned, cols % 256 == 0) into blocks tiling each row, in the
 * layouts the expert kernels read: dst gets n_mats*rows*cols/256 blocks of
 * 84 (Q2_K, dst 4-byte aligned), 66 (IQ2_XXS, 2-byte aligned) or 144 bytes
 * (Q4_K, 16-byte aligned), or n_mats*rows*cols/32 blocks of 34 bytes (Q8_0,
 * 2-byte aligned; d = max|x|/127 per 32 values, importance unused).  Q4_K
 * is the Q2_K procedure on 32-value sub-blocks with 4-bit codes and 6-bit
 * scale/min nibbles (the Q4 layers of the mixed stacks, DS4C2 sec. 10).
 * importance: device, nullable for Q2_K and Q4_K (every weight 1: the plain
 * encoder), required for IQ2_XXS; matrix m's weights are importance[m * imp_stride + c]
 * for column c (imp_stride 0: one vector for every matrix; otherwise a
 * multiple of 4, normally cols: the n_expert x n_columns packing), 16-byte
 * aligned.  grid and iq2_map (IQ2_XXS only): the grid as for
 * ds4moe_iq2_map_build and the map built from it.  Non-finite values or
 * weights, and negative weights, set DS4MOE_FAULT_BAD_INPUT in the status
 * word of ws (>= 256 bytes); the blocks are then unspecified.  Returns
 * DS4MOE_EINVAL for a bad type, pointer, alignment or shape.  Asynchronous.
 */
ds4moe_status ds4moe_quantize(int32_t qtype, const float* src, int64_t n_mats, int64_t rows,
                              int64_t cols, const float* importance, int64_t imp_stride,
                              const uint8_t* grid, const void* iq2_map, void* dst, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/*
 * Fallback importance (DS4C2 sec. 8): out[m][c] = sum_r src[m][r][c]^2 for
 * n_mats fp32 matrices [rows][cols] (device), accumulated in fp32 in row
 * order with fused multiply-adds.  out: device, n_mats * cols floats.
 */
ds4moe_status ds4moe_column_energy(const float* src, int64_t n_mats, int64_t rows, int64_t cols,
                                   float* out, hipStream_t stream);

/*
 * Waits for `stream`, reads and clears the workspace status word.  Returns
 * DS4MOE_OK if no fault bit was set, DS4MOE_EDATA otherwise; *faults
 * (nullable, host) receives the bits.
 */
ds4moe_status ds4moe_check(void* ws, hipStream_t stream, uint32_t* faults);

const char* ds4moe_status_string(ds4moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* DS4MOE_H */
