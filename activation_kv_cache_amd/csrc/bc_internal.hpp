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

constexpr int kGemvTile = 128;   // output columns per work-group (16 lanes x 8)
constexpr int kGemvThreads = 256;

enum GemvMode : int { MAIN_PARTIAL = 0, MAIN_BF16 = 1, MAIN_F32_ARGMAX = 2 };
enum FinishKind : int { FIN_BF16 = 0, FIN_QKV = 1, FIN_RESID = 2, FIN_SWIGLU = 3 };

struct GemvPlan {
  int n_tiles;
  int n_splits;
  int rows_per_split;
  size_t partial_bytes;   // n_splits * d_out fp32
};
GemvPlan plan_gemv(int d_out, int k);

struct GemvParams {
  const uint16_t* wt;
  int tiled;              // 1: tile-major [tile][d_in][tile width]; 0: plain [d_in][d_out]
  int d_in, d_out;
  const uint16_t* x;
  const int32_t* idx;
  int k;
  int rows_per_split, n_splits, n_tiles;
  float* partial;         // MAIN_PARTIAL: [n_splits][d_out]
  uint16_t* y;            // MAIN_BF16
  float* yf;              // MAIN_F32_ARGMAX
  float* tile_max;
  int32_t* tile_arg;
};
int launch_gemv_main(int mode, const GemvParams& p, hipStream_t s);

struct FinishParams {
  const float* partial;
  int n_splits, d_out;
  uint16_t* y;                  // bf16 output (d_out, or d_ff for SwiGLU)
  const uint16_t* resid;        // FIN_RESID: optional residual
  const uint16_t* norm_gain;    // FIN_RESID: RMSNorm gain of the next input (optional)
  float eps;
  uint16_t* x_next;             // FIN_RESID: RMSNorm output
  int sel_k;                    // top-k of the next input when 0 < sel_k < n
  int32_t* idx_next;
  // FIN_QKV
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* summary;
  int n_heads, n_kv_heads, head_dim, n_cap, pos;
  double log2_theta;
  // FIN_SWIGLU
  int d_ff;
};
int launch_finish(int kind, const FinishParams& p, hipStream_t s);
int launch_argmax_finish(const float* tile_max, const int32_t* tile_arg, int n_tiles, int32_t* token, hipStream_t s);

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int n_cap;
  const int32_t* idx;
  int n_sel, n_heads, n_kv_heads, head_dim, n_splits;
  float scale_log2;
  float* m;
  float* l;
  float* o;
};
int launch_attn_partial(const AttnParams& p, hipStream_t s);

struct ReduceParams {
  const float* m;
  const float* l;
  const float* o;
  int n_heads, n_splits, head_dim;
  uint16_t* out;
};
int launch_attn_reduce(const ReduceParams& p, hipStream_t s);
// merge and, when 0 < k < n_heads*head_dim, the top-k of the merged output
int launch_attn_reduce_select(const ReduceParams& p, int k, int32_t* idx_out, hipStream_t s);

struct KvSelectParams {
  const uint16_t* q;
  const uint16_t* summary;
  int nb_cap, n_ctx, n_heads, n_kv_heads, head_dim;
  bc_kv_budget_info bud;
  float* scores;          // [n_kv_heads][n_cand]
  int32_t* idx_out;       // [n_kv_heads][t_sel]
};
int launch_kv_score_select(const KvSelectParams& p, hipStream_t s);

int launch_norm_select(const uint16_t* h, const uint16_t* g, int d, float eps, uint16_t* x_out, int k,
                       int32_t* idx_out, hipStream_t s);
int launch_select(const uint16_t* x, int n, int k, int32_t* idx_out, hipStream_t s);
int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);

bool valid_head_dim(int hd);
bool valid_group(int g);

}  // namespace bc
