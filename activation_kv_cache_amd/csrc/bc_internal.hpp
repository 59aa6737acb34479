// bc_internal.hpp -- host-side declarations shared by libbc's sources:
// error reporting, launch plans and the internal kernel launchers that
// bc_decode_layer chains on one stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bc.h"

namespace bc {

int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Rotary cos/sin of the current position, pair i = (i, i + head_dim/2),
// computed on the host in double (angle pos * theta^(-2i/head_dim)) and
// rounded to float; passed to the kernels by value.
constexpr int kRopeMaxPairs = 64;   // head_dim <= 128
struct RopeTable {
  float c[kRopeMaxPairs];
  float s[kRopeMaxPairs];
};
void rope_table(int pos, double theta, int head_dim, RopeTable* t);

constexpr int kGemvTile = 128;      // output columns per work-group (16 lanes x 8)
constexpr int kGemvThreads = 1024;  // 64 row slots of 16 lanes
constexpr int kGemvMaxRows = 4096;  // rows (list positions) per work-group
constexpr int kGemvFusedMaxIn = 16384;  // inputs a work-group normalises / selects itself

// Where a GEMV work-group gets its input rows and values:
//   IN_LIST  x and an optional ascending channel list are given;
//   IN_NORM  x = bf16(RMSNorm(h) * gain) is formed in the prologue, then
//            (k < d_in) the exact top-k of |x| is selected there too;
//   IN_SEL   x is given and (k < d_in) its top-k is selected in the prologue.
//   IN_NORM_SUM  as IN_NORM, with h itself formed first from the fp32 chunk
//            partials of the GEMV before it plus a residual:
//            h = bf16(sum of chunks in chunk order + resid), the arithmetic
//            of FIN_RESID; the first work-group stores h (h_out).  This folds
//            a residual finish kernel into the next GEMV (d_in <= 4096).
//   IN_ATTN  dense only: x is the attention output, formed for the chunk's
//            own channels from the split-K partials (m, l, o) in the combine
//            order of the reduce kernel; this folds the reduce into the o
//            GEMV.  The first tile's work-groups store their channels of x
//            (x_out), which together cover it.
// Every work-group of a launch forms the same x and the same selection; the
// first one also stores them (x_out, idx_out) when asked.
enum GemvIn : int { IN_LIST = 0, IN_NORM = 1, IN_SEL = 2, IN_NORM_SUM = 3, IN_ATTN = 4 };
// What the main kernel stores: fp32 partials per chunk of rows, or (one
// chunk) bf16 y, the SwiGLU of a gate|up tile, or fp32 y + per-tile argmax.
enum GemvOut : int { OUT_PARTIAL = 0, OUT_BF16 = 1, OUT_SWIGLU = 2, OUT_ARGMAX = 3 };
enum FinishKind : int { FIN_BF16 = 0, FIN_QKV = 1, FIN_RESID = 2, FIN_SWIGLU = 3, FIN_ARGMAX = 4, FIN_NONE = 5 };

struct GemvPlan {
  int n_tiles;
  int n_splits;
  int rows_per_split;
  size_t partial_bytes;   // n_splits * d_out fp32
};
// single: one chunk of rows if it fits a work-group (for OUT_BF16 / SWIGLU /
// ARGMAX epilogues); max_splits > 0 caps the chunk count where the rows
// allow it (a work-group takes at most kGemvMaxRows)
GemvPlan plan_gemv(int d_out, int k, bool single = false, int max_splits = 0);
bool gemv_fused_input_ok(int d_in);
bool gemv_sum_input_ok(int d_in);   // IN_NORM_SUM supports this d_in
// IN_ATTN supports a dense GEMV of d_in = heads * head_dim inputs over this
// many attention splits
constexpr int kAttnFoldMaxSplits = 32;
bool gemv_attn_fold_ok(int d_in, int d_out, int head_dim, int attn_splits);

struct GemvParams {
  const uint16_t* wt;
  int tiled;              // 1: tile-major [tile][d_in][tile width]; 0: plain [d_in][d_out]
  int d_in, d_out;
  const uint16_t* x;      // IN_LIST, IN_SEL: bf16 [d_in]
  const int32_t* idx;     // IN_LIST: [k] or NULL
  const uint16_t* h;      // IN_NORM: bf16 [d_in]; IN_NORM_SUM: the residual
  const uint16_t* gain;   // IN_NORM, IN_NORM_SUM: bf16 [d_in]
  const float* sum_partial;   // IN_NORM_SUM: [sum_splits][d_in] fp32
  int sum_splits;
  uint16_t* h_out;        // IN_NORM_SUM: h (first work-group)
  const float* am;        // IN_ATTN: split partials m, l [heads][a_splits], o [heads][a_splits][a_hd]
  const float* al;
  const float* ao;
  int a_splits, a_hd;
  float eps;
  uint16_t* x_out;        // IN_NORM / IN_SEL: optional copy of x (first work-group)
  int32_t* idx_out;       // IN_NORM / IN_SEL: optional copy of the selection
  int k;
  int rows_per_split, n_splits, n_tiles;
  float* partial;         // OUT_PARTIAL: [n_splits][d_out]
  uint16_t* y;            // OUT_BF16: [d_out]; OUT_SWIGLU: [d_out / 2]
  float* yf;              // OUT_ARGMAX
  float* tile_max;
  int32_t* tile_arg;
  unsigned long long* clk;   // phase clocks of the launch (set by launch_gemv; NULL in the library itself)
};
int launch_gemv(int in, int out, const GemvParams& p, hipStream_t s);

struct FinishParams {
  const float* partial;
  int n_splits, d_out;
  uint16_t* y;                  // bf16 output (d_out, or d_ff for SwiGLU)
  const uint16_t* resid;        // FIN_RESID: residual added to the sum
  // FIN_QKV
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* summary;
  int n_heads, n_kv_heads, head_dim, n_cap, pos;
  RopeTable rope;
  // FIN_SWIGLU
  int d_ff;
  // FIN_ARGMAX
  float* yf;
  float* tile_max;
  int32_t* tile_arg;
};
int launch_finish(int kind, const FinishParams& p, hipStream_t s);
// work-groups of a FIN_ARGMAX launch (entries of tile_max / tile_arg)
int finish_argmax_groups(int d_out);
int launch_argmax_finish(const float* tile_max, const int32_t* tile_arg, int n_tiles, int32_t* token, hipStream_t s);

// Where the partial pass gets q and its list of tokens.
//   Q_GLOBAL   q bf16 [n_heads][head_dim] is given;
//   Q_PARTIAL  q, k, v of the current token come from the qkv GEMV chunk
//              partials (rotary at pos, bf16 rounding); the work-group whose
//              range holds list position pos (dense list, pos = n_sel - 1)
//              appends k, v at cache slot pos and attends to them from LDS.
//   L_DENSE    tokens 0..n_sel-1;  L_IDX  an index list [n_kv_heads][n_sel];
//   L_SCORES   the list sinks | top-k_blk scored blocks | window: each split
//              selects the block ranks its slice needs from the block scores
//              in its prologue, or (blk given) copies them from the kept
//              blocks' candidate indices in rank order.
enum AttnQ : int { Q_GLOBAL = 0, Q_PARTIAL = 1 };
enum AttnList : int { L_DENSE = 0, L_IDX = 1, L_SCORES = 2 };
constexpr int kAttnMaxCand = 256 * 8;    // candidate blocks one attention work-group selects from
constexpr int kAttnMaxRanks = 1024;      // block ranks one split may need

struct AttnParams {
  const uint16_t* q;
  uint16_t* k_cache;      // written only by the appending work-group
  uint16_t* v_cache;
  int n_cap;
  const int32_t* idx;
  int n_sel, n_heads, n_kv_heads, head_dim, n_splits;
  float scale_log2;
  float* m;
  float* l;
  float* o;
  // Q_PARTIAL
  const float* qkv_partial;   // [qkv_splits][qkv_out]
  int qkv_splits, qkv_out;
  int pos;
  RopeTable rope;
  uint16_t* q_out;            // optional bf16 copy of q
  uint16_t* summary;          // optional: (min, max) of block pos/16 refreshed by the appending work-group
  // L_SCORES
  const float* scores;        // [n_kv_heads][scores_stride]
  int scores_stride;
  const int32_t* blk;         // optional: [n_kv_heads][k_blk] kept candidates by rank
  bc_kv_budget_info bud;
  int n_ctx;
  int32_t* idx_out;           // optional: the list [n_kv_heads][n_sel] (each split writes its slice)
  unsigned long long* clk;    // phase clocks of the launch (set by launch_attn_partial; NULL in the library itself)
};
int launch_attn_partial(int q_mode, int list_mode, const AttnParams& p, hipStream_t s);
// whether a scored list fits the attention kernel (candidates, ranks per split)
bool attn_scored_list_ok(const bc_kv_budget_info& bud, int n_splits);
// whether its prologue selection is cheap enough (few candidates per
// thread); otherwise a selection kernel supplies the ranks (AttnParams::blk)
bool attn_prologue_select_ok(const bc_kv_budget_info& bud);

struct ReduceParams {
  const float* m;
  const float* l;
  const float* o;
  int n_heads, n_splits, head_dim;
  uint16_t* out;
};
int launch_attn_reduce(const ReduceParams& p, hipStream_t s);

struct KvSelectParams {
  const uint16_t* q;
  uint16_t* summary;
  int nb_cap, n_ctx, n_heads, n_kv_heads, head_dim;
  bc_kv_budget_info bud;
  float* scores;          // [n_kv_heads][scores_stride]
  int scores_stride;
  int32_t* idx_out;       // [n_kv_heads][t_sel], or NULL
  int32_t* blk_out;       // optional: [n_kv_heads][k_blk] kept candidates by rank
  // q from the qkv GEMV partials (rotary at pos): the first work-group of
  // each KV head also stores q, appends k, v at slot pos and refreshes the
  // summary of block pos/16 (valid when that block is never a candidate)
  const float* qkv_partial;
  int qkv_splits, qkv_out, pos, n_cap;
  RopeTable rope;
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int score_bpg;          // candidate blocks per scoring work-group (set by launch_kv_score)
};
// scores, then the list (one work-group per KV head)
int launch_kv_score_select(const KvSelectParams& p, hipStream_t s);
// scores only (q given or from the partials, with the append)
int launch_kv_score(const KvSelectParams& p, hipStream_t s);
// the list (idx_out) and / or the kept candidates by rank (blk_out) from the
// scores
int launch_kv_block_select(const KvSelectParams& p, hipStream_t s);

// The masked-attention dense baseline (bc_masked.hip): out bf16 [H][D].
size_t masked_attn_workspace(int n_cap, int n_heads, int head_dim);
int launch_masked_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int n_cap, int n_ctx,
                       int n_heads, int n_kv_heads, int head_dim, float scale, uint16_t* out, void* ws,
                       hipStream_t s);

int launch_select(const uint16_t* x, int n, int k, int32_t* idx_out, hipStream_t s);
// one selection per sequence of a batch: x [batch][x_stride], idx_out [batch][k]
int launch_select_batch(const uint16_t* x, int n, int k, int32_t* idx_out, int batch, int x_stride, hipStream_t s);
// the batched union GEMV (bc_gemv_batch.hip) without the ABI checks: bf16 y
// or (y == NULL) fp32 yf [batch][d_out]
int run_gemv_batch(const uint16_t* wt, int tiled, int d_in, int d_out, const uint16_t* x, const int32_t* idx, int k,
                   int batch, uint16_t* y, float* yf, int32_t* n_union_out, void* ws, size_t ws_bytes, hipStream_t s);
int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);

bool valid_head_dim(int hd);
bool valid_group(int g);

}  // namespace bc
