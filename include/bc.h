/*
 * bc.h -- C ABI of libbc: one decode step of one sequence on an MI355X
 * (gfx950): activation-sparse projection GEMV and split-K grouped-query
 * decode attention over a KV cache that is read densely or through an
 * attention-scored selection of sinks, history blocks and a recent window.
 *
 * Source of the method: "Where Activation Sparsity and KV-Cache Sparsity
 * Cross in LLM Decoding" (ByteCross), GitHub README page.  Each entry point
 * names the README section that defines what it computes.
 *
 * Conventions (all entry points)
 *   - bf16 values are uint16_t bit patterns.  Every data pointer is a DEVICE
 *     pointer owned by the caller, 16-byte aligned, contiguous in the layout
 *     stated; the library never keeps a pointer after the call returns.
 *   - No entry point allocates, frees or synchronises.  All work is enqueued
 *     on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *   - Return BC_OK (0) or a negative error code.  Arguments are checked on the
 *     host before anything is enqueued; on error nothing is enqueued and
 *     bc_last_error() returns a message (thread-local).  No exception crosses
 *     the ABI.
 *   - Index contents are not checked on the device: out-of-range channel or
 *     token ids are undefined behaviour.
 *   - Every count (k, T_sel, split sizes) is a function of host-known
 *     scalars, so no call reads anything back from the device.
 *   - Workspaces: a workspace is caller-owned device memory whose size comes
 *     from the matching *_workspace_bytes query.  It must be cleared once with
 *     bc_workspace_init after allocation; every call leaves it ready for the
 *     next one.  Calls that share one workspace must not overlap in time.
 */
#ifndef BC_H
#define BC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BC_ABI_VERSION 6

enum {
  BC_OK = 0,
  BC_ERR_INVALID = -1,     /* NULL pointer, bad size, k out of range       */
  BC_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, group size... */
  BC_ERR_WORKSPACE = -3,   /* workspace smaller than the query returned    */
  BC_ERR_HIP = -4          /* a HIP launch or runtime call failed          */
};

/* Decoder dimensions (README "Quick start": the config fields the byte
 * account reads).  head_dim * n_heads must equal d (README FAQ).
 * Supported here: head_dim in {64, 128}; n_heads / n_kv_heads in {1,2,4,8}. */
typedef struct {
  int n_layers, d, d_ff, vocab, n_heads, n_kv_heads, head_dim;
} bc_model_dims;

/* KV policy (README "What it does in one picture": the kept entries are the
 * first tokens, a share of the older history and the newest tokens).  r_kv >= 1 reads the
 * whole cache.  block must be 16 (the summary granularity). */
typedef struct {
  double r_kv;
  int sinks;
  int window;
  int block;
} bc_kv_policy;

/* Sizes of one KV selection, all host-computable:
 *   T = min(n, floor(r_kv*n + 1/2)); sinks' = min(sinks, T);
 *   window' = min(window, T - sinks'); candidates = the 16-aligned blocks that
 *   lie wholly in [sinks', n - window'); k_blk = min(floor((T - sinks' -
 *   window')/16), candidates); T_sel = sinks' + window' + 16*k_blk.
 *   For r_kv >= 1: T_sel = n and nothing is scored. */
typedef struct {
  int t_sel, k_blk, n_cand, b_lo, sinks, window;
} bc_kv_budget_info;

int bc_abi_version(void);
const char* bc_last_error(void);

/* Number of kept channels: floor(r_p*d_in + 1/2) clamped to [1, d_in];
 * r_p >= 1 keeps all d_in.  Returns the count (>0) or BC_ERR_INVALID. */
int bc_channel_keep(double r_p, int d_in);

/* Fills *out (see bc_kv_budget_info).  Returns BC_OK or BC_ERR_INVALID. */
int bc_kv_budget(int n_ctx, const bc_kv_policy* pol, bc_kv_budget_info* out);

/* Clears `bytes` bytes of a workspace with a fill kernel (no memset node,
 * so it may be captured in a graph). */
int bc_workspace_init(void* ws, size_t bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* a1. Channel selection (README "What it does in one picture"; "Timing and
 * quality on a GPU": activation sparsity on all seven projections).
 * Exact top-k of |x| over x[0..d_in): the key of channel i is bits(x_i) &
 * 0x7FFF; larger key first, equal keys by lower index; -0 and +0 tie.
 * idx_out[0..k) receives the kept channels in ascending order.
 * 1 <= k <= d_in <= 65536.  x: bf16 [d_in]; idx_out: int32 [k]. */
int bc_select_channels(const uint16_t* x, int d_in, int k, int32_t* idx_out, void* stream);

/* a2. Sparse projection GEMV (README "What it does": the activations select
 * the weight columns that are read).  y[o] = sum_{j<k} W^T[idx_j][o] * x[idx_j]
 * with fp32 accumulation, rounded to bf16 (nearest even).
 *   wt  bf16 [d_in][d_out]  W transposed: row i is input channel i's weights
 *   x   bf16 [d_in]
 *   idx int32 [k] ascending channel ids, or NULL for the dense GEMV (k = d_in)
 *   y   bf16 [d_out]
 * d_out % 8 == 0.  ws/ws_bytes from bc_sparse_gemv_workspace_bytes(d_out, k).
 * The sum over channels is split into fixed chunks and added in a fixed
 * order, so results are deterministic run to run. */
size_t bc_sparse_gemv_workspace_bytes(int d_out, int k);
int bc_sparse_gemv(const uint16_t* wt, int d_in, int d_out, const uint16_t* x, const int32_t* idx,
                   int k, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* The same GEMV (same kernel, same result bits) over W^T in the tile-major
 * layout of bc_pack_weight_tiles, the layout bc_decode_layer reads. */
int bc_sparse_gemv_tiled(const uint16_t* wt_packed, int d_in, int d_out, const uint16_t* x, const int32_t* idx,
                         int k, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* a2 for a batch (README "Quick start", crossover_batch: a batch reads the
 * projection weights once for the union of the channels its sequences keep;
 * the key-value bytes stay per sequence).  Sequence b keeps its own k
 * channels and gets its own sparse GEMV:
 *   y[b][o] = sum_{j<k} W^T[idx[b][j]][o] * x[b][idx[b][j]]   (fp32, then bf16)
 * The matrix rows read are the union U of the batch's channel lists, each
 * once; |U| / d_in is the union keep of crossover_batch.
 *   wt     bf16 W^T [d_in][d_out], row-major (tiled = 0) or in the tile-major
 *          layout of bc_pack_weight_tiles (tiled = 1)
 *   x      bf16 [batch][d_in]
 *   idx    int32 [batch][k], each row ascending channel ids, or NULL for the
 *          dense GEMV of every sequence (k = d_in); ids outside [0, d_in)
 *          are ignored
 *   y      bf16 [batch][d_out]
 *   n_union_out  optional device int32 that receives |U| (NULL: not written)
 * 1 <= batch <= 4, d_in <= 16384, d_out % 8 == 0, and for the row-major
 * layout d_in * d_out < 2^32 (else BC_ERR_UNSUPPORTED).  ws/ws_bytes from
 * bc_sparse_gemv_batch_workspace_bytes(d_in, d_out, k, batch) (0 for sizes
 * out of range); it holds per-range row counts and partial sums and is
 * overwritten.  The order of the sums is fixed (U ascending, in fixed
 * channel ranges added in range order), so results are deterministic run to
 * run; they equal bc_sparse_gemv's up to fp32 rounding order. */
size_t bc_sparse_gemv_batch_workspace_bytes(int d_in, int d_out, int k, int batch);
int bc_sparse_gemv_batch(const uint16_t* wt, int tiled, int d_in, int d_out, const uint16_t* x, const int32_t* idx,
                         int k, int batch, uint16_t* y, int32_t* n_union_out, void* ws, size_t ws_bytes,
                         void* stream);

/* a4. Attention-scored KV selection (README "What it does in one picture":
 * the first tokens, a share of the older history and the newest tokens are
 * kept), the history scored per 16-token block by an upper
 * bound of the query-key product built from per-block key minima and maxima.
 * For KV head g and candidate block b (see bc_kv_budget_info), with the
 * group's query heads j:
 *   P_d = adjacent-pair tree over j of (q_{j,d} > 0 ? q_{j,d} : 0)
 *   N_d = adjacent-pair tree over j of (q_{j,d} > 0 ? 0 : q_{j,d})
 *   t_d = fma(kmax_{b,d}, P_d, kmin_{b,d} * N_d)   (the product kmin*N rounded first)
 *   a_p = (t_{4p} + t_{4p+1}) + (t_{4p+2} + t_{4p+3})
 *   s_{g,b} = adjacent-pair tree over p = 0..head_dim/4-1 of a_p
 * (adjacent-pair tree: v_i <- v_{2i} + v_{2i+1} until one value remains;
 * fp32 in exactly this order).  In real arithmetic (kmax >= kmin)
 * t_d = sum_j max(q_{j,d}*kmax_{b,d}, q_{j,d}*kmin_{b,d}), so s bounds
 * sum_j q_j . k_t from above for every token t of the block.  The k_blk highest scores are kept (equal
 * scores: lower block); idx_out[g] = sinks, kept blocks' tokens and the
 * window, ascending.
 *   q        bf16 [n_heads][head_dim] post-rotary query; query head j reads
 *            KV head j / (n_heads/n_kv_heads)
 *   summary  bf16 [n_kv_heads][nb_cap][head_dim][2]  (min, max) per dim
 *   idx_out  int32 [n_kv_heads][T_sel]
 *   scores_out  optional fp32 [n_kv_heads][n_cand] (candidate order)
 * Requires r_kv < 1 (the dense case needs no list).  ws from
 * bc_kv_score_select_workspace_bytes. */
size_t bc_kv_score_select_workspace_bytes(int n_ctx, int n_kv_heads, const bc_kv_policy* pol);
int bc_kv_score_select(const uint16_t* q, const uint16_t* summary, int nb_cap, int n_ctx,
                       int n_heads, int n_kv_heads, int head_dim, const bc_kv_policy* pol,
                       int32_t* idx_out, float* scores_out, void* ws, size_t ws_bytes, void* stream);

/* Per-block key summaries of a pre-filled cache (setup, not timed):
 * for every 16-token block holding tokens below n_ctx, per dim the min and
 * max over those tokens.  k_cache bf16 [n_kv_heads][n_cap][head_dim];
 * summary bf16 [n_kv_heads][n_cap/16][head_dim][2].  n_cap % 16 == 0. */
int bc_build_kv_summary(const uint16_t* k_cache, int n_kv_heads, int n_cap, int head_dim, int n_ctx,
                        uint16_t* summary, void* stream);

/* a4 (select once).  The README's timing harness also runs the KV branch as
 * "sel": the scored selection made once and copied into a buffer of its own
 * and then read by the same dense attention kernel every step (README
 * "Timing and quality on a GPU"; "API at a glance": select_and_compact).
 * This is the gather: for every KV head g and t < t_sel,
 *   k_out[g][t][:] = k_cache[g][idx[g][t]][:],  v_out likewise.
 *   k_cache, v_cache  bf16 [n_kv_heads][n_cap][head_dim]
 *   idx     int32 [n_kv_heads][t_sel] token ids (a list from bc_kv_score_select)
 *   k_out, v_out  bf16 [n_kv_heads][n_cap_out][head_dim]; rows >= t_sel untouched
 * t_sel <= n_cap_out.  Ids outside [0, n_cap) are clamped (never read out of
 * the cache).  The output must not overlap the input. */
int bc_kv_compact(const uint16_t* k_cache, const uint16_t* v_cache, int n_cap, int n_kv_heads, int head_dim,
                  const int32_t* idx, int t_sel, uint16_t* k_out, uint16_t* v_out, int n_cap_out, void* stream);

/* a4 (select once, SnapKV form).  The README's KV branch follows SnapKV with
 * one selection after prefill (README FAQ "How is this different from TEAL
 * and SnapKV?"); the selection is then gathered (bc_kv_compact) and read by
 * the same dense split-K attention every step ("Timing and quality on a
 * GPU"; "API at a glance": select_and_compact).  For KV head g, the
 * observation rows are the w_obs queries of the last positions
 * p_i = n_ctx - w_obs + i in each of the group's query heads j:
 *   A_{i,j,t} = softmax over t <= p_i of scale * (q_obs[i][j] . k_t),
 *               scale = 1/sqrt(head_dim);
 *   vote_t   = sum_i sum_j A_{i,j,t}                      (t < n_ctx)
 *   score_t  = (1/pool_kernel) * sum of vote_u over |u - t| <= pool_kernel/2
 *              (votes outside [0, n_ctx) are 0)
 * Budget (tokens, host-computable by bc_kv_snap_t_sel):
 *   T = min(n, floor(r_kv*n + 1/2)); sinks' = min(sinks, T);
 *   window' = min(window, T - sinks'); the k = T - sinks' - window' highest
 *   float32 scores among tokens [sinks', n - window') are kept (equal scores:
 *   lower token); T_sel = T.
 * idx_out[g] = sinks', kept tokens, window', ascending.  policy->block is
 * not used (token granularity).  The logits are computed with bf16 matrix
 * instructions and float32 accumulation; softmax, votes and pooling in
 * float32.
 *   q_obs     bf16 [w_obs][n_heads][head_dim]  post-rotary observation queries
 *   k_cache   bf16 [n_kv_heads][n_cap][head_dim]
 *   idx_out   int32 [n_kv_heads][T_sel]
 *   scores_out  optional fp32 [n_kv_heads][n_ctx]: score_t of every token
 * Requires r_kv < 1, 1 <= w_obs <= n_ctx <= n_cap, w_obs * (n_heads /
 * n_kv_heads) a multiple of 32 and at most 256 (BC_ERR_UNSUPPORTED
 * otherwise), pool_kernel odd in [1, 63], q_obs and k_cache 16-byte aligned,
 * ws 256-byte aligned, ws_bytes from bc_kv_snap_select_workspace_bytes.  Run
 * once per layer after prefill; not part of the decode step. */
int bc_kv_snap_t_sel(int n_ctx, const bc_kv_policy* pol);
size_t bc_kv_snap_select_workspace_bytes(int n_ctx, int n_heads, int n_kv_heads, int w_obs);
int bc_kv_snap_select(const uint16_t* q_obs, int w_obs, const uint16_t* k_cache, int n_cap, int n_ctx, int n_heads,
                      int n_kv_heads, int head_dim, const bc_kv_policy* pol, int pool_kernel, int32_t* idx_out,
                      float* scores_out, void* ws, size_t ws_bytes, void* stream);

/* a5. Split-K decode attention, partial pass (README "Overview": one split-K
 * kernel serves the dense and every sparse mode).  For
 * query head j (KV head g = j / (n_heads/n_kv_heads)) and split s covering
 * list positions [s*c, min(n_sel, (s+1)*c)), c = ceil(n_sel/n_splits):
 *   z_t = scale * (q_j . k_t); m = max z; l = sum e^(z-m); o = sum e^(z-m) v_t
 * (m in natural-log units, o unnormalised; an empty split gives (-inf,0,0)).
 *   q       bf16 [n_heads][head_dim]
 *   k_cache, v_cache  bf16 [n_kv_heads][n_cap][head_dim]
 *   idx     int32 [n_kv_heads][n_sel] token ids, or NULL for tokens 0..n_sel-1
 *   m, l    fp32 [n_heads][n_splits];  o  fp32 [n_heads][n_splits][head_dim]
 * 1 <= n_splits <= 4096. */
int bc_splitk_attn_partial(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int n_cap,
                           const int32_t* idx, int n_sel, int n_heads, int n_kv_heads, int head_dim,
                           int n_splits, float scale, float* m, float* l, float* o, void* stream);

/* a6. Merge of the split partials (README "Overview", split-K attention):
 * M = max_s m_s; out = sum_s o_s e^(m_s-M) / sum_s l_s e^(m_s-M), rounded to
 * bf16; all splits empty gives 0.  out bf16 [n_heads][head_dim].  The fp32
 * order is fixed (the denominator over 256 thread slots and a fixed
 * cross-lane sum per wave, the numerator in 256/head_dim groups of consecutive splits
 * with fma in split order), and bc_decode_layer's dense o projection, which
 * merges the splits in its own prologue, follows the same order: its
 * attention output equals this call's on the same partials, bit for bit. */
int bc_splitk_reduce(const float* m, const float* l, const float* o, int n_heads, int n_splits,
                     int head_dim, uint16_t* out, void* stream);

/* The masked-attention dense baseline (README FAQ "A KV method reports a
 * speedup above its byte bound": a dense baseline built on masked attention
 * makes a KV policy look faster than one built on split-K attention does; the
 * abstract puts the factor near five).  Decode attention as a plain masked attention
 * over a preallocated cache computes it, for every query head j (KV head
 * g = j / (n_heads/n_kv_heads)):
 *   z_t = scale * (q_j . k_t) for every cache slot t < n_cap, -inf for
 *         t >= n_ctx (the mask);  p = softmax(z) over all n_cap slots;
 *   out_j = sum over all n_cap slots of p_t v_t, rounded to bf16.
 * The scores and weights ([n_heads][n_cap] fp32) go through the workspace
 * between the kernels, and each query head reads its KV head's rows itself.
 * In real arithmetic it equals softmax attention over tokens 0..n_ctx-1.
 * Slots n_ctx..n_cap-1 are read and must hold finite values.
 *   q  bf16 [n_heads][head_dim]; k_cache, v_cache bf16 [n_kv_heads][n_cap][head_dim]
 *   out bf16 [n_heads][head_dim]
 * n_cap % 16 == 0, 1 <= n_ctx <= n_cap; ws 256-byte aligned, ws_bytes from
 * bc_masked_attn_workspace_bytes. */
size_t bc_masked_attn_workspace_bytes(int n_cap, int n_heads, int head_dim);
int bc_masked_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int n_cap, int n_ctx,
                   int n_heads, int n_kv_heads, int head_dim, float scale, uint16_t* out, void* ws, size_t ws_bytes,
                   void* stream);

/* Split count the library picks for n_sel listed tokens (used when a step
 * passes n_splits = 0). */
int bc_attn_default_splits(int n_sel, int n_kv_heads);

/* ---------------------------------------------------------------------- */
/* a7. One decoder layer of the decode step (README "Timing and quality on a
 * GPU": TEAL on all seven projections, the cache read through split-K
 * attention; the layer glue is the plain Llama reading):
 *   x1 = RMSNorm(h)*g_attn; S1 = top-k(x1); [q k v] = W_qkv[:,S1] x1[S1];
 *   rotary (rotate-half, theta) on q and k at position n_ctx-1; k, v written
 *   to slot n_ctx-1 and that block's (min, max) summary recomputed;
 *   L = KV selection (r_kv < 1) or tokens 0..n_ctx-1; a = attention(q, L);
 *   S2 = top-k(a); h1 = h + W_o[:,S2] a[S2]; x2 = RMSNorm(h1)*g_mlp;
 *   S3 = top-k(x2); f = SiLU(W_gate x2) * (W_up x2) over S3;
 *   S4 = top-k(f); h = h1 + W_down[:,S4] f[S4].
 * k = bc_channel_keep(r_p, d_in) per GEMV input; r_p >= 1 is dense. */
/* Weights of a layer are W^T in the tile-major layout of
 * bc_pack_weight_tiles (gate and up together through bc_pack_gate_up). */
typedef struct {
  const uint16_t* w_qkv;   /* packed W^T, d_in d, d_out n_heads*hd + 2*n_kv_heads*hd  (q | k | v) */
  const uint16_t* w_o;     /* packed W^T, d_in n_heads*hd, d_out d */
  const uint16_t* w_gu;    /* from bc_pack_gate_up, d_in d, d_out 2*d_ff */
  const uint16_t* w_down;  /* packed W^T, d_in d_ff, d_out d */
  const uint16_t* g_attn;  /* bf16 [d] */
  const uint16_t* g_mlp;   /* bf16 [d] */
  uint16_t* k_cache;       /* bf16 [n_kv_heads][n_cap][hd] */
  uint16_t* v_cache;       /* bf16 [n_kv_heads][n_cap][hd] */
  uint16_t* kv_summary;    /* bf16 [n_kv_heads][n_cap/16][hd][2]; may be NULL when r_kv >= 1 */
  int n_cap;               /* multiple of 16 */
} bc_layer;

/* Optional copies of every stage (device buffers, any may be NULL). */
typedef struct {
  uint16_t* x1;       /* [d] */
  int32_t* idx_qkv;   /* [k_d] */
  uint16_t* q;        /* [n_heads][hd] post-rotary */
  uint16_t* k;        /* [n_kv_heads][hd] post-rotary */
  uint16_t* v;        /* [n_kv_heads][hd] */
  int32_t* idx_kv;    /* [n_kv_heads][T_sel] */
  uint16_t* a;        /* [n_heads*hd] */
  int32_t* idx_o;     /* [k_d] */
  uint16_t* h_mid;    /* [d] */
  uint16_t* x2;       /* [d] */
  int32_t* idx_gu;    /* [k_d] */
  uint16_t* hff;      /* [d_ff] */
  int32_t* idx_down;  /* [k_ff] */
  float* attn_m;      /* [n_heads][n_splits] split-K partials of the attention */
  float* attn_l;      /* [n_heads][n_splits] */
  float* attn_o;      /* [n_heads][n_splits][hd] */
} bc_layer_taps;

typedef struct {
  int n_ctx;           /* tokens attended, the current one included (1..n_cap) */
  double r_p;          /* projection keep; >= 1 dense */
  bc_kv_policy kv;     /* r_kv >= 1 dense */
  int n_splits;        /* attention splits; 0 = bc_attn_default_splits */
  double rope_theta;   /* e.g. 500000 */
  double rms_eps;      /* e.g. 1e-5 */
  const bc_layer_taps* taps;  /* optional */
  /* Optional: the dense baseline with masked attention (bc_masked_attn) in
   * place of split-K attention, its workspace of bc_masked_attn_workspace_bytes
   * (n_cap, n_heads, head_dim) bytes given here; NULL = split-K attention.
   * Requires r_kv >= 1. */
  void* masked_ws;
  size_t masked_ws_bytes;
} bc_step;

size_t bc_layer_workspace_bytes(const bc_model_dims* dims, int max_ctx, int max_splits);
int bc_decode_layer(const bc_model_dims* dims, const bc_layer* layer, const bc_step* step,
                    uint16_t* hidden, void* ws, size_t ws_bytes, void* stream);

/* a8. One whole decode step (README "Timing and quality on a GPU": a step
 * is every layer with all seven projections and the cache read, then the
 * LM head, whose weights are in the step's bytes -- README "Quick start",
 * the 1.60x bound).  For each of layers[0..n_layers) the work of
 * bc_decode_layer (same kernels, same results); the last layer's output
 * goes through RMSNorm(h) * g_final and the dense LM head into logits fp32
 * [vocab], and token[0] = argmax (lowest index on ties).  Across layer
 * boundaries the next layer's RMSNorm and channel top-k are produced by the
 * previous layer's last kernel, so a step launches one kernel fewer per
 * layer than n_layers separate bc_decode_layer calls.  step->taps is
 * ignored.  w_head: W_head^T packed by bc_pack_weight_tiles (d_in d, d_out
 * vocab).  ws from bc_step_workspace_bytes. */
size_t bc_step_workspace_bytes(const bc_model_dims* dims, int max_ctx, int max_splits);
int bc_decode_step(const bc_model_dims* dims, const bc_layer* layers, int n_layers, const uint16_t* g_final,
                   const uint16_t* w_head, const bc_step* step, uint16_t* hidden, float* logits, int32_t* token,
                   void* ws, size_t ws_bytes, void* stream);

/* The step of bc_decode_step without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus ws and
 * ws_bytes), same kernels, same result bits.  The workspace is a static
 * device array of BC_STATIC_SCRATCH_BYTES (16 MiB) inside the library, which
 * each GPU the library runs on holds until the process ends; this call
 * allocates and frees nothing.  A step whose workspace
 * (bc_step_workspace_bytes) is larger fails with BC_ERR_WORKSPACE before
 * anything is enqueued (at Llama-3.1-8B dims with the default splits that is
 * a context above about 440K tokens).  The first call on a device, with that
 * device current, looks up the array's address and enqueues one fill kernel
 * on `stream` that clears it.  Every call on a GPU shares that GPU's array
 * and leaves in it what the last call wrote: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be ordered by the
 * caller. */
#define BC_STATIC_SCRATCH_BYTES (16u << 20)
int bc_decode_step_noalloc(const bc_model_dims* dims, const bc_layer* layers, int n_layers, const uint16_t* g_final,
                           const uint16_t* w_head, const bc_step* st, uint16_t* hidden, float* logits,
                           int32_t* token, void* stream);

/* A batch of up to four sequences that share the weights (README "Quick
 * start" and "Usage": crossover_batch -- a batch reads the projection
 * weights once for the union of the channels its sequences keep, and the
 * key-value bytes once per sequence).  layers[b] (b < batch) holds the
 * shared weights (every entry the same pointers) and sequence b's own cache
 * and summaries; every sequence attends to step->n_ctx tokens.  Per
 * sequence the layer computes what bc_decode_layer does (its own channel
 * selections, rotary, append, KV selection and attention), with the
 * projections of the whole batch read through one union GEMV each
 * (bc_sparse_gemv_batch): hidden [batch][d] in and out.  Every value is
 * rounded to bf16 where bc_decode_layer rounds it (the projections hand fp32
 * sums on), so results equal bc_decode_layer's up to the fp32 order of the
 * sums over the kept channels.  taps: NULL or [batch] (attn_m/l/o are not
 * written).
 * step->masked_ws must be NULL.  ws from bc_layer_batch_workspace_bytes. */
size_t bc_layer_batch_workspace_bytes(const bc_model_dims* dims, int batch, int max_ctx, int max_splits);
int bc_decode_layer_batch(const bc_model_dims* dims, const bc_layer* layers, int batch, const bc_step* step,
                          uint16_t* hidden, const bc_layer_taps* taps, void* ws, size_t ws_bytes, void* stream);

/* A whole decode step for a batch: layers [n_layers][batch] (layer-major),
 * then per sequence the final RMSNorm and the dense LM head (its weights
 * read once for the batch), logits fp32 [batch][vocab], tokens [batch]
 * (argmax, lowest index on ties).  ws from bc_layer_batch_workspace_bytes
 * with the same dims (vocab included). */
int bc_decode_step_batch(const bc_model_dims* dims, const bc_layer* layers, int n_layers, int batch,
                         const uint16_t* g_final, const uint16_t* w_head, const bc_step* step, uint16_t* hidden,
                         float* logits, int32_t* tokens, void* ws, size_t ws_bytes, void* stream);

/* Tile-major re-layout of a W^T matrix for bc_decode_layer and bc_lm_head
 * (setup, not timed): the columns are cut into tiles of 128 (the last one
 * narrower, w_t columns); tile t stores its d_in rows contiguously, row i at
 * packed + t*128*d_in + i*w_t.  A GEMV work-group that owns one tile and a
 * chunk of rows then reads one contiguous block.  wt bf16 [d_in][d_out],
 * packed bf16 (d_in*d_out elements, not aliasing wt); d_out % 8 == 0. */
int bc_pack_weight_tiles(const uint16_t* wt, int d_in, int d_out, uint16_t* packed, void* stream);

/* Packs W_gate^T and W_up^T (each bf16 [d][d_ff]) for bc_decode_layer: the
 * columns are first interleaved per tile -- gate columns [64t, 64t + w) then
 * up columns [64t, 64t + w), w = min(64, d_ff - 64t) -- and the result is laid
 * out tile-major as bc_pack_weight_tiles does (d_in d, d_out 2*d_ff).
 * (setup, not timed) */
int bc_pack_gate_up(const uint16_t* w_gate_t, const uint16_t* w_up_t, int d, int d_ff, uint16_t* w_gu,
                    void* stream);

/* a8 tail. Final RMSNorm and the dense LM head of the step (the LM head is
 * in the step's bytes: README "Quick start", the 1.60x bound):
 * logits = W_head (RMSNorm(h)*g), token = argmax (lowest index on ties).
 *   w_head_t: W_head^T (d_in d, d_out vocab) packed by bc_pack_weight_tiles;
 *   logits fp32 [vocab]; token int32 [1]. */
size_t bc_lm_head_workspace_bytes(const bc_model_dims* dims);
int bc_lm_head(const bc_model_dims* dims, const uint16_t* hidden, const uint16_t* g_final,
               const uint16_t* w_head_t, float* logits, int32_t* token, double rms_eps,
               void* ws, size_t ws_bytes, void* stream);

/* Measurement helper, not a step of the method: reads bytes from src once,
 * as 256 work-groups of 1024 lanes that each stream one contiguous share
 * with the hot kernels' 16-byte non-temporal loads, two in flight per lane,
 * and writes one checksum word per work-group to sink[256] (so the loads
 * are not dead).  Timed, it gives the practical HBM read ceiling reported
 * beside the 8 TB/s peak.  bytes: a positive multiple of 4 MiB (256 * 1024
 * * 16); src 16-byte aligned.  Errors: BC_ERR_INVALID for a NULL pointer,
 * a misaligned src or a size that is not such a multiple. */
int bc_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Measurement helpers, not steps of the method: per-phase clocks of the GEMV
 * and attention kernels.  Only the instrumented build of this library
 * (libbc_clk.so, compiled with -DBC_PHASE_CLOCKS; same kernels plus clock
 * reads) records them; the library itself returns BC_ERR_UNSUPPORTED from
 * all three and its kernels take no clock reads.
 * bc_phase_clocks_begin registers buf (device memory, 8-byte aligned, bytes
 * long; NULL stops recording) and forgets earlier launches; each later GEMV
 * or attention-partial launch then takes the next 16 64-bit entries per
 * work-group of it, while they fit, and its work-group g stores at
 * entries [16 g, 16 g + 16) of its slice: the 100 MHz real-time counter at
 * its start and end, the shader clock at its start, at phase ends and at
 * its end, its XCC id and hardware id (which phase each entry holds is
 * listed in the kernel's source).  A launch recorded during graph capture
 * writes its slice at every replay.  The caller owns buf and reads it after
 * the kernels end.
 * bc_phase_clocks_count: the number of launches recorded since the last
 * begin (or a negative error code).
 * bc_phase_clocks_info(i, out7): launch i as out7 = {kind (1 GEMV, 2
 * attention), a, b, c, d, work-groups, first entry}; a..d are, for a GEMV,
 * (input mode | output mode << 8, d_in, d_out, k) and, for attention, (q
 * mode | list mode << 8, listed tokens, splits, KV heads).  Errors:
 * BC_ERR_INVALID for i out of range or a NULL out7. */
int bc_phase_clocks_begin(void* buf, size_t bytes);
int bc_phase_clocks_count(void);
int bc_phase_clocks_info(int i, long long* out7);

#ifdef __cplusplus
}
#endif

#endif /* BC_H */
