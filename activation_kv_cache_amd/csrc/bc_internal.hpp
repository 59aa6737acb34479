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

constexpr int kGemvTile = 512;   // output columns per work-group (64 lanes x 8)
constexpr int kGemvThreads = 256;

enum Epi : int { EPI_BF16 = 0, EPI_F32_ARGMAX = 1, EPI_RESID = 2, EPI_QKV = 3, EPI_SWIGLU = 4 };
enum Tail : int { TAIL_NONE = 0, TAIL_SELECT = 1, TAIL_NORM_SELECT = 2, TAIL_ARGMAX = 3 };

struct GemvPlan {
  int n_tiles;
  int n_splits;
  int rows_per_split;
  size_t counter_bytes;   // (n_tiles + 1) uint32, 256-aligned
  size_t partial_bytes;   // n_splits * d_out fp32 when n_splits > 1
};
GemvPlan plan_gemv(int d_out, int k);

struct GemvParams {
  const uint16_t* wt;
  int d_in, d_out;
  const uint16_t* x;
  const int32_t* idx;
  int k;
  int rows_per_split, n_splits, n_tiles;
  float* partial;
  uint32_t* counters;     // n_tiles + 1, zero on entry, zero on exit
  // epilogues
  uint16_t* y;
  float* yf;
  const uint16_t* resid;
  uint16_t* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  uint16_t* summary;
  int n_heads, n_kv_heads, head_dim, n_cap, pos;
  float pad0;
  double theta;
  int d_ff;
  float* tile_max;
  int32_t* tile_arg;
  int32_t* token_out;
  // tail (run once by the last work-group to finish)
  int tail;
  const uint16_t* tail_in;
  int tail_n;
  const uint16_t* tail_gain;
  float tail_eps;
  uint16_t* tail_x_out;
  int tail_k;
  int32_t* tail_idx_out;
};
int launch_gemv(int epi, const GemvParams& p, hipStream_t s);

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
  uint32_t* counters;     // 1 word; only with a select tail
  int tail_k;             // select top-k of out (n_heads*head_dim) when 0 < tail_k < n
  int32_t* tail_idx_out;
};
int launch_attn_reduce(const ReduceParams& p, hipStream_t s);

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
