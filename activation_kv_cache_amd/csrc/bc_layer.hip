// bc_layer.hip -- one decoder layer of the decode step, the LM head, and the
// small entry points of libbc (errors, budgets, workspace, packing).
//
// bc_decode_layer enqueues, on one stream and with no host synchronisation
// (kernel boundaries are the only cross-work-group synchronisation):
//   k_gemv<IN_NORM>, k_finish_qkv   x1 = RMSNorm(h) * g_attn and S1 = top-k(x1)
//                          in every work-group's prologue; q, k, v over S1;
//                          rotary; append k, v at slot n-1; refresh that
//                          block's (min, max) summary
//   k_kv_score, k_kv_block_select   KV list (r_kv < 1 only)
//   k_attn_partial, k_attn_reduce   split-K attention -> a
//   k_gemv<IN_SEL>, k_finish_resid  S2 = top-k(a) in the prologue;
//                          h1 = h + W_o a over S2.  A dense o GEMV
//                          (k_gemv<IN_ATTN>) forms its chunk of a from the
//                          split partials itself and the reduce is skipped
//   k_gemv<IN_NORM, OUT_SWIGLU>     x2 = RMSNorm(h1) * g_mlp, S3 = top-k(x2);
//                          f = SiLU(gate) * up over S3 (one chunk per tile)
//   k_gemv<IN_SEL>, k_finish_resid  S4 = top-k(f); h = h1 + W_down f over S4
// Every launch size depends only on host-known scalars.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {
thread_local char g_err[512] = "";
}  // namespace

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(BC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return BC_OK;
}

bool valid_head_dim(int hd) { return hd == 64 || hd == 128; }
bool valid_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

void rope_table(int pos, double theta, int head_dim, RopeTable* t) {
  const int half = head_dim / 2;
  for (int i = 0; i < kRopeMaxPairs; ++i) {
    if (i < half) {
      const double ang = double(pos) * pow(theta, -2.0 * double(i) / double(head_dim));
      t->c[i] = float(cos(ang));
      t->s[i] = float(sin(ang));
    } else {
      t->c[i] = 1.0f;
      t->s[i] = 0.0f;
    }
  }
}

namespace {

// Streaming read of a contiguous share per work-group, two 16-byte
// non-temporal loads in flight per lane (bc_stream_read).
constexpr int kReadGroups = 256;
constexpr int kReadThreads = 1024;
__global__ __launch_bounds__(kReadThreads) void k_stream_read(const uint4* src, size_t n16_per_group, uint32_t* sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* base = reinterpret_cast<const u32x4*>(src) + size_t(blockIdx.x) * n16_per_group;
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i < n16_per_group; i += 2 * kReadThreads) {
    const size_t j = i + kReadThreads;
    const u32x4 a = __builtin_nontemporal_load(base + i);
    const u32x4 b = j < n16_per_group ? __builtin_nontemporal_load(base + j) : u32x4{0u, 0u, 0u, 0u};
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w);
  }
  // one word per work-group (wave 0's sum); every lane's loads run either way
  acc = wave_sum_u32(acc);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ void k_fill_zero(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0)
    for (size_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

// Tile-major re-layout of W^T [d_in][d_out]: column tile t (kGemvTile wide,
// the last one narrower) stores its d_in rows contiguously, each row as wide
// as the tile.  With gate_up, the source columns are first interleaved per
// tile: gate columns [64t, 64t + w) then up columns [64t, 64t + w),
// w = min(64, d_ff - 64t), from two [d_in][d_ff] matrices (d_out = 2 d_ff).
__global__ __launch_bounds__(256) void k_pack_tiles(const uint16_t* src, const uint16_t* src_up, int d_in,
                                                   int d_out, uint16_t* out) {
  const int row = blockIdx.x;
  const int d_ff = d_out / 2;
  for (int c = threadIdx.x; c < d_out; c += 256) {
    const int t = c / kGemvTile, off = c % kGemvTile;
    const int tw = min(kGemvTile, d_out - t * kGemvTile);
    uint16_t v;
    if (src_up == nullptr) {
      v = src[size_t(row) * d_out + c];
    } else {
      const int half = kGemvTile / 2;
      const int w = min(half, d_ff - t * half);
      v = off < w ? src[size_t(row) * d_ff + t * half + off] : src_up[size_t(row) * d_ff + t * half + off - w];
    }
    out[size_t(t) * kGemvTile * d_in + size_t(row) * tw + off] = v;
  }
}

// ------------------------------------------------------------ layer layout
struct LayerLayout {
  size_t partial, partial2, x1, idx_qkv, q, scores, blk, idx_kv, m, l, o, a, idx_o, h_mid, x2, idx_gu, hff, idx_down;
  size_t total;
};

// Chunk partials: the q/k/v and gate|up GEMVs use one buffer, the o and
// down GEMVs (whose partials the next GEMV's prologue folds into the
// residual stream) another, so a prologue never reads a buffer its own
// launch writes.
size_t gemv_partial_max(const bc_model_dims& m, bool od) {
  const int qkv = m.n_heads * m.head_dim + 2 * m.n_kv_heads * m.head_dim;
  size_t mx = 0;
  const int outs[4] = {qkv, m.d, 2 * m.d_ff, m.d};
  const int ins[4] = {m.d, m.n_heads * m.head_dim, m.d, m.d_ff};
  for (int i = 0; i < 4; ++i) {
    if (od != (i == 1 || i == 3)) continue;
    GemvPlan pl = plan_gemv(outs[i], ins[i], i == 2);
    if (pl.partial_bytes > mx) mx = pl.partial_bytes;
  }
  return mx;
}

LayerLayout layer_layout(const bc_model_dims& m, int n_ctx, int n_splits) {
  LayerLayout L;
  size_t off = 0;
  auto take = [&off](size_t bytes) { size_t o = off; off += align_up(bytes > 0 ? bytes : 1, 256); return o; };
  const int hd = m.head_dim, H = m.n_heads, Hkv = m.n_kv_heads;
  const int nb = (n_ctx + 15) / 16;
  L.partial = take(gemv_partial_max(m, false));
  L.partial2 = take(gemv_partial_max(m, true));
  L.x1 = take(size_t(m.d) * 2);
  L.idx_qkv = take(size_t(m.d) * 4);
  L.q = take(size_t(H) * hd * 2);
  L.scores = take(size_t(Hkv) * nb * 4);
  L.blk = take(size_t(Hkv) * (nb + 1) * 4);
  L.idx_kv = take(size_t(Hkv) * n_ctx * 4);
  L.m = take(size_t(H) * n_splits * 4);
  L.l = take(size_t(H) * n_splits * 4);
  L.o = take(size_t(H) * n_splits * hd * 4);
  L.a = take(size_t(H) * hd * 2);
  L.idx_o = take(size_t(H) * hd * 4);
  L.h_mid = take(size_t(m.d) * 2);
  L.x2 = take(size_t(m.d) * 2);
  L.idx_gu = take(size_t(m.d) * 4);
  L.hff = take(size_t(m.d_ff) * 2);
  L.idx_down = take(size_t(m.d_ff) * 4);
  L.total = off;
  return L;
}

int check_dims(const bc_model_dims* m) {
  if (!m) return set_error(BC_ERR_INVALID, "NULL dims");
  if (m->d <= 0 || m->d_ff <= 0 || m->n_heads <= 0 || m->n_kv_heads <= 0 || m->head_dim <= 0)
    return set_error(BC_ERR_INVALID, "dims: non-positive size");
  if (m->n_heads * m->head_dim != m->d) return set_error(BC_ERR_INVALID, "dims: n_heads*head_dim != d");
  if (m->n_heads % m->n_kv_heads != 0) return set_error(BC_ERR_INVALID, "dims: n_heads %% n_kv_heads != 0");
  if (!valid_head_dim(m->head_dim)) return set_error(BC_ERR_UNSUPPORTED, "dims: head_dim %d", m->head_dim);
  if (!valid_group(m->n_heads / m->n_kv_heads)) return set_error(BC_ERR_UNSUPPORTED, "dims: group size");
  if (m->d % 8 != 0 || m->d_ff % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "dims: d and d_ff must be multiples of 8");
  if (!gemv_fused_input_ok(m->d) || !gemv_fused_input_ok(m->d_ff))
    return set_error(BC_ERR_UNSUPPORTED, "dims: d and d_ff must be at most %d", kGemvFusedMaxIn);
  return BC_OK;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int copy_tap(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (!dst || bytes == 0) return BC_OK;
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? BC_OK : set_error(BC_ERR_HIP, "tap copy: %s", hipGetErrorString(e));
}

}  // namespace

int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  k_fill_zero<<<dim3(unsigned(blocks)), dim3(256), 0, s>>>(static_cast<uint4*>(ptr), n16,
                                                           static_cast<uint8_t*>(ptr) + n16 * 16, ntail);
  return check_launch("k_fill_zero");
}

}  // namespace bc

using namespace bc;

extern "C" int bc_abi_version(void) { return BC_ABI_VERSION; }
extern "C" const char* bc_last_error(void) { return g_err; }

extern "C" int bc_channel_keep(double r_p, int d_in) {
  if (d_in <= 0 || !(r_p > 0.0)) return set_error(BC_ERR_INVALID, "bc_channel_keep: r_p=%g d_in=%d", r_p, d_in);
  if (r_p >= 1.0) return d_in;
  long long k = static_cast<long long>(floor(r_p * double(d_in) + 0.5));
  if (k < 1) k = 1;
  if (k > d_in) k = d_in;
  return static_cast<int>(k);
}

extern "C" int bc_workspace_init(void* ws, size_t bytes, void* stream) {
  if (bytes == 0) return BC_OK;
  if (!ws) return set_error(BC_ERR_INVALID, "bc_workspace_init: NULL workspace");
  if (reinterpret_cast<uintptr_t>(ws) & 15) return set_error(BC_ERR_INVALID, "bc_workspace_init: ws not 16-byte aligned");
  return launch_fill_zero(ws, bytes, static_cast<hipStream_t>(stream));
}

extern "C" int bc_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  constexpr size_t kUnit = size_t(kReadGroups) * kReadThreads * 16;
  if (!src || !sink) return set_error(BC_ERR_INVALID, "bc_stream_read: NULL pointer");
  if (reinterpret_cast<uintptr_t>(src) & 15) return set_error(BC_ERR_INVALID, "bc_stream_read: src not 16-byte aligned");
  if (bytes == 0 || bytes % kUnit != 0)
    return set_error(BC_ERR_INVALID, "bc_stream_read: %zu bytes is not a positive multiple of %zu", bytes, kUnit);
  k_stream_read<<<dim3(kReadGroups), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), bytes / 16 / kReadGroups, sink);
  return check_launch("k_stream_read");
}

extern "C" int bc_select_channels(const uint16_t* x, int d_in, int k, int32_t* idx_out, void* stream) {
  if (!x || !idx_out) return set_error(BC_ERR_INVALID, "bc_select_channels: NULL pointer");
  if (d_in < 1 || d_in > 65536) return set_error(BC_ERR_INVALID, "bc_select_channels: d_in=%d", d_in);
  if (k < 1 || k > d_in) return set_error(BC_ERR_INVALID, "bc_select_channels: k=%d outside [1, %d]", k, d_in);
  return launch_select(x, d_in, k, idx_out, static_cast<hipStream_t>(stream));
}

extern "C" int bc_pack_gate_up(const uint16_t* w_gate_t, const uint16_t* w_up_t, int d, int d_ff, uint16_t* w_gu,
                               void* stream) {
  if (!w_gate_t || !w_up_t || !w_gu) return set_error(BC_ERR_INVALID, "bc_pack_gate_up: NULL pointer");
  if (d <= 0 || d_ff <= 0 || d_ff % 8 != 0) return set_error(BC_ERR_INVALID, "bc_pack_gate_up: d=%d d_ff=%d", d, d_ff);
  k_pack_tiles<<<dim3(d), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(w_gate_t, w_up_t, d, 2 * d_ff, w_gu);
  return check_launch("k_pack_tiles");
}

extern "C" int bc_pack_weight_tiles(const uint16_t* wt, int d_in, int d_out, uint16_t* packed, void* stream) {
  if (!wt || !packed) return set_error(BC_ERR_INVALID, "bc_pack_weight_tiles: NULL pointer");
  if (d_in <= 0 || d_out <= 0 || d_out % 8 != 0)
    return set_error(BC_ERR_INVALID, "bc_pack_weight_tiles: d_in=%d d_out=%d", d_in, d_out);
  if (wt == packed) return set_error(BC_ERR_INVALID, "bc_pack_weight_tiles: in-place packing is not supported");
  k_pack_tiles<<<dim3(d_in), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(wt, nullptr, d_in, d_out, packed);
  return check_launch("k_pack_tiles");
}

extern "C" size_t bc_layer_workspace_bytes(const bc_model_dims* dims, int max_ctx, int max_splits) {
  if (check_dims(dims) != BC_OK || max_ctx < 1 || max_splits < 1) return 0;
  return layer_layout(*dims, max_ctx, max_splits).total;
}

namespace {

// What a projection GEMV reads: IN_NORM forms x = RMSNorm(v) * gain, IN_SEL
// takes x = v; with k < d_in the prologue also selects the top-k of |x|.
// IN_NORM_SUM first forms v = bf16(chunk sums of sum_partial + resid) and
// stores it at h_out.
struct ProjIn {
  int mode;
  const uint16_t* v;    // IN_NORM_SUM: the residual
  const uint16_t* gain;
  float eps;
  uint16_t* x_out;      // optional copy of x
  int32_t* idx_out;     // optional copy of the selection
  const float* sum_partial = nullptr;
  int sum_splits = 0;
  uint16_t* h_out = nullptr;
  const float* am = nullptr;   // IN_ATTN: attention split partials
  const float* al = nullptr;
  const float* ao = nullptr;
  int a_splits = 0, a_hd = 0;
};

// A hidden state not yet stored: h = bf16(chunk sums of partial + resid),
// left by a GEMV for the next GEMV's prologue to form.
struct Pending {
  const float* partial;
  int n_splits;
  const uint16_t* resid;
};

ProjIn norm_input(const uint16_t* h, const Pending* pend, uint16_t* h_out, const uint16_t* gain, float eps,
                  uint16_t* x_out, int32_t* idx_out) {
  ProjIn in{IN_NORM, h, gain, eps, x_out, idx_out};
  if (pend) {
    in.mode = IN_NORM_SUM;
    in.v = pend->resid;
    in.sum_partial = pend->partial;
    in.sum_splits = pend->n_splits;
    in.h_out = h_out;
  }
  return in;
}

// One projection: main kernel and, with several chunks, its finish.  The
// gate|up GEMV (FIN_SWIGLU) runs as one chunk per tile when it fits, with
// the SwiGLU in the main kernel's epilogue.  FIN_NONE leaves the chunk
// partials for the next kernel (their count in *n_splits).
int run_gemv(const uint16_t* wt, int d_in, int d_out, int k, const ProjIn& in, float* partial, int fin_kind,
             FinishParams f, hipStream_t s, int* n_splits = nullptr, int max_splits = 0) {
  const bool swiglu = fin_kind == FIN_SWIGLU;
  const GemvPlan pl = plan_gemv(d_out, k, swiglu, max_splits);
  if (n_splits) *n_splits = pl.n_splits;
  GemvParams p{};
  p.wt = wt; p.tiled = 1; p.d_in = d_in; p.d_out = d_out; p.k = k;
  if (in.mode == IN_NORM || in.mode == IN_NORM_SUM) {
    p.h = in.v; p.gain = in.gain; p.eps = in.eps;
    p.sum_partial = in.sum_partial; p.sum_splits = in.sum_splits; p.h_out = in.h_out;
  } else if (in.mode == IN_ATTN) {
    p.am = in.am; p.al = in.al; p.ao = in.ao; p.a_splits = in.a_splits; p.a_hd = in.a_hd;
  } else {
    p.x = in.v;
  }
  p.x_out = in.x_out; p.idx_out = in.idx_out;
  p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
  p.partial = partial;
  if (swiglu && pl.n_splits == 1) {
    p.y = f.y;
    return launch_gemv(in.mode, OUT_SWIGLU, p, s);
  }
  int rc = launch_gemv(in.mode, OUT_PARTIAL, p, s);
  if (rc != BC_OK || fin_kind == FIN_NONE) return rc;
  f.partial = partial;
  f.n_splits = pl.n_splits;
  f.d_out = d_out;
  return launch_finish(fin_kind, f, s);
}

// Final RMSNorm (in the GEMV prologue), dense LM head and argmax.  With a
// pending hidden state the prologue forms it first and stores it at hidden.
int run_head(const bc_model_dims& m, uint16_t* hidden, const Pending* pend, const uint16_t* g_final,
             const uint16_t* w_head, float eps, float* logits, int32_t* token, float* partial, float* tile_max,
             int32_t* tile_arg, hipStream_t s) {
  const GemvPlan pl = plan_gemv(m.vocab, m.d, true);
  GemvParams p{};
  p.wt = w_head; p.tiled = 1; p.d_in = m.d; p.d_out = m.vocab; p.k = m.d;
  p.h = hidden; p.gain = g_final; p.eps = eps;
  int in_mode = IN_NORM;
  if (pend) {
    in_mode = IN_NORM_SUM;
    p.h = pend->resid; p.sum_partial = pend->partial; p.sum_splits = pend->n_splits; p.h_out = hidden;
  }
  p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
  p.yf = logits; p.tile_max = tile_max; p.tile_arg = tile_arg; p.partial = partial;
  int rc;
  if (pl.n_splits == 1) {
    if ((rc = launch_gemv(in_mode, OUT_ARGMAX, p, s)) != BC_OK) return rc;
    return launch_argmax_finish(tile_max, tile_arg, pl.n_tiles, token, s);
  }
  if ((rc = launch_gemv(in_mode, OUT_PARTIAL, p, s)) != BC_OK) return rc;
  FinishParams f{};
  f.partial = partial; f.n_splits = pl.n_splits; f.d_out = m.vocab;
  f.yf = logits; f.tile_max = tile_max; f.tile_arg = tile_arg;
  if ((rc = launch_finish(FIN_ARGMAX, f, s)) != BC_OK) return rc;
  return launch_argmax_finish(tile_max, tile_arg, finish_argmax_groups(m.vocab), token, s);
}

// Workspace of the LM head: chunk partials (only when d exceeds one chunk)
// and the per-tile argmax candidates.
struct HeadLayout { size_t partial, tile_max, tile_arg, total; };
HeadLayout head_layout(const bc_model_dims& m, size_t off = 0) {
  const GemvPlan pl = plan_gemv(m.vocab, m.d, true);
  const int n_cand = pl.n_tiles > finish_argmax_groups(m.vocab) ? pl.n_tiles : finish_argmax_groups(m.vocab);
  HeadLayout L;
  auto take = [&off](size_t bytes) { size_t o = off; off += align_up(bytes > 0 ? bytes : 1, 256); return o; };
  L.partial = take(pl.n_splits > 1 ? pl.partial_bytes : 256);
  L.tile_max = take(size_t(n_cand) * 4);
  L.tile_arg = take(size_t(n_cand) * 4);
  L.total = off;
  return L;
}

}  // namespace

namespace {

int check_layer(const bc_layer* ly, const bc_step* st) {
  if (!ly->w_qkv || !ly->w_o || !ly->w_gu || !ly->w_down || !ly->g_attn || !ly->g_mlp || !ly->k_cache ||
      !ly->v_cache)
    return set_error(BC_ERR_INVALID, "NULL layer pointer");
  if (ly->n_cap <= 0 || ly->n_cap % 16 != 0) return set_error(BC_ERR_INVALID, "n_cap %% 16 != 0");
  if (st->n_ctx < 1 || st->n_ctx > ly->n_cap)
    return set_error(BC_ERR_INVALID, "n_ctx=%d outside [1, n_cap=%d]", st->n_ctx, ly->n_cap);
  if (st->kv.r_kv < 1.0 && !ly->kv_summary) return set_error(BC_ERR_INVALID, "r_kv < 1 needs kv_summary");
  return BC_OK;
}

// The masked-attention baseline's workspace against the layer's cache.
int check_masked(const bc_model_dims& m, const bc_layer* ly, const bc_step* st) {
  if (!st->masked_ws) return BC_OK;
  const size_t need = masked_attn_workspace(ly->n_cap, m.n_heads, m.head_dim);
  if (st->masked_ws_bytes < need)
    return set_error(BC_ERR_WORKSPACE, "masked attention workspace %zu < %zu", st->masked_ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(st->masked_ws) & 255) return set_error(BC_ERR_INVALID, "masked_ws not 256-byte aligned");
  return BC_OK;
}

int check_step(const bc_step* st) {
  if (!(st->r_p > 0.0)) return set_error(BC_ERR_INVALID, "r_p must be > 0");
  if (!(st->rms_eps >= 0.0) || !(st->rope_theta > 0.0)) return set_error(BC_ERR_INVALID, "eps/theta out of range");
  if (st->n_splits < 0 || st->n_splits > 4096) return set_error(BC_ERR_INVALID, "n_splits=%d", st->n_splits);
  if (st->masked_ws && st->kv.r_kv < 1.0)
    return set_error(BC_ERR_UNSUPPORTED, "masked attention is the dense baseline: it needs r_kv >= 1");
  return BC_OK;
}

int step_splits(const bc_model_dims& m, const bc_step* st, const bc_kv_budget_info& bud) {
  const int n_sel = st->kv.r_kv < 1.0 ? bud.t_sel : st->n_ctx;
  return st->n_splits > 0 ? st->n_splits : bc_attn_default_splits(n_sel, m.n_kv_heads);
}

// One decoder layer.  pin: the layer's input is pending (formed by the q/k/v
// GEMV's prologue, which stores it at hidden); pout: leave the output pending
// (the down GEMV's chunk partials plus h1) instead of storing it at hidden.
int layer_body(const bc_model_dims& m, const bc_layer* ly, const bc_step* st, const bc_kv_budget_info& bud,
               int n_splits, uint16_t* hidden, const Pending* pin, Pending* pout, void* ws, const LayerLayout& L,
               hipStream_t s) {
  int rc;
  const int hd = m.head_dim, H = m.n_heads, Hkv = m.n_kv_heads;
  const bool kv_sparse = st->kv.r_kv < 1.0;
  const int n_sel = kv_sparse ? bud.t_sel : st->n_ctx;
  const bool sparse = st->r_p < 1.0;
  const int k_d = bc_channel_keep(st->r_p, m.d);
  const int k_ff = bc_channel_keep(st->r_p, m.d_ff);
  const int qkv_out = H * hd + 2 * Hkv * hd;
  const int pos = st->n_ctx - 1;
  float* partial = at<float>(ws, L.partial);
  float* partial2 = at<float>(ws, L.partial2);
  const float eps = float(st->rms_eps);
  int32_t* idx_qkv = sparse ? at<int32_t>(ws, L.idx_qkv) : nullptr;
  int32_t* idx_o = sparse ? at<int32_t>(ws, L.idx_o) : nullptr;
  int32_t* idx_gu = sparse ? at<int32_t>(ws, L.idx_gu) : nullptr;
  int32_t* idx_down = sparse ? at<int32_t>(ws, L.idx_down) : nullptr;
  uint16_t* h_mid = at<uint16_t>(ws, L.h_mid);
  uint16_t* a = at<uint16_t>(ws, L.a);
  uint16_t* hff = at<uint16_t>(ws, L.hff);

  // x1 = RMSNorm(h), S1 (GEMV prologue); q, k, v from its chunk partials.
  // Dense list: the attention kernel applies the rotary, appends k, v and
  // refreshes the block summary itself.  Scored list: the scoring kernel
  // does that (unless the window is empty, when the current block may be a
  // candidate: then a finish kernel does it first), and every attention
  // work-group selects the blocks of its own slice of the list.
  const ProjIn qkv_in = norm_input(hidden, pin, hidden, ly->g_attn, eps, at<uint16_t>(ws, L.x1), idx_qkv);
  RopeTable rope;
  rope_table(pos, st->rope_theta, hd, &rope);
  int qkv_splits = 0;
  const bool masked = st->masked_ws != nullptr;   // the masked-attention dense baseline
  const bool fused_score = kv_sparse && (bud.window > 0 || bud.k_blk == 0);
  const bool scored_attn = kv_sparse && attn_scored_list_ok(bud, n_splits);
  // many candidates: one 1024-lane work-group per KV head ranks them once
  // (a kernel boundary) instead of every attention work-group in its prologue
  const bool rank_kernel = scored_attn && bud.k_blk > 0 && !attn_prologue_select_ok(bud);
  KvSelectParams kp{};
  if (kv_sparse) {
    kp.summary = ly->kv_summary; kp.nb_cap = ly->n_cap / 16; kp.n_ctx = st->n_ctx;
    kp.n_heads = H; kp.n_kv_heads = Hkv; kp.head_dim = hd; kp.bud = bud;
    kp.scores = at<float>(ws, L.scores); kp.scores_stride = bud.n_cand > 0 ? bud.n_cand : 1;
    kp.idx_out = at<int32_t>(ws, L.idx_kv);
  }
  if ((kv_sparse && !fused_score) || masked) {
    FinishParams f{};
    f.q_out = at<uint16_t>(ws, L.q); f.k_cache = ly->k_cache; f.v_cache = ly->v_cache; f.summary = ly->kv_summary;
    f.n_heads = H; f.n_kv_heads = Hkv; f.head_dim = hd; f.n_cap = ly->n_cap; f.pos = pos; f.rope = rope;
    if ((rc = run_gemv(ly->w_qkv, m.d, qkv_out, k_d, qkv_in, partial, FIN_QKV, f, s)) != BC_OK) return rc;
    kp.q = at<uint16_t>(ws, L.q);
    if (kv_sparse && (rc = launch_kv_score(kp, s)) != BC_OK) return rc;
  } else {
    if ((rc = run_gemv(ly->w_qkv, m.d, qkv_out, k_d, qkv_in, partial, FIN_NONE, FinishParams{}, s, &qkv_splits,
                       kQkvMaxChunks)) != BC_OK)
      return rc;
    if (kv_sparse) {
      kp.qkv_partial = partial; kp.qkv_splits = qkv_splits; kp.qkv_out = qkv_out; kp.pos = pos; kp.n_cap = ly->n_cap;
      kp.rope = rope; kp.q_out = at<uint16_t>(ws, L.q); kp.k_cache = ly->k_cache; kp.v_cache = ly->v_cache;
      if ((rc = launch_kv_score(kp, s)) != BC_OK) return rc;
    }
  }
  if (kv_sparse && !scored_attn && (rc = launch_kv_block_select(kp, s)) != BC_OK) return rc;
  if (rank_kernel) {
    KvSelectParams kb = kp;
    kb.idx_out = nullptr;
    kb.blk_out = at<int32_t>(ws, L.blk);
    if ((rc = launch_kv_block_select(kb, s)) != BC_OK) return rc;
  }

  // attention; a dense o GEMV folds the reduce into its prologue
  const bool fold_reduce = !masked && k_d == H * hd && gemv_attn_fold_ok(H * hd, m.d, hd, n_splits);
  if (masked) {
    const float scale = float(1.0 / sqrt(double(hd)));
    if ((rc = launch_masked_attn(at<uint16_t>(ws, L.q), ly->k_cache, ly->v_cache, ly->n_cap, st->n_ctx, H, Hkv, hd,
                                 scale, a, st->masked_ws, s)) != BC_OK)
      return rc;
  } else {
    AttnParams p{};
    p.k_cache = ly->k_cache; p.v_cache = ly->v_cache; p.n_cap = ly->n_cap;
    p.n_sel = n_sel; p.n_heads = H; p.n_kv_heads = Hkv; p.head_dim = hd; p.n_splits = n_splits;
    // softmax scale 1/sqrt(head_dim), in the arithmetic of bc_splitk_attn_partial
    p.scale_log2 = float(1.0 / sqrt(double(hd))) * 1.4426950408889634f;
    p.m = at<float>(ws, L.m); p.l = at<float>(ws, L.l); p.o = at<float>(ws, L.o);
    ReduceParams r{};
    r.m = p.m; r.l = p.l; r.o = p.o; r.n_heads = H; r.n_splits = n_splits; r.head_dim = hd; r.out = a;
    if (kv_sparse) {
      p.q = at<uint16_t>(ws, L.q);
      if (scored_attn) {
        p.scores = kp.scores; p.scores_stride = kp.scores_stride; p.bud = bud; p.n_ctx = st->n_ctx;
        p.blk = rank_kernel ? at<int32_t>(ws, L.blk) : nullptr;
        p.idx_out = st->taps ? at<int32_t>(ws, L.idx_kv) : nullptr;
        if ((rc = launch_attn_partial(Q_GLOBAL, L_SCORES, p, s)) != BC_OK) return rc;
      } else {
        p.idx = at<int32_t>(ws, L.idx_kv);
        if ((rc = launch_attn_partial(Q_GLOBAL, L_IDX, p, s)) != BC_OK) return rc;
      }
    } else {
      p.qkv_partial = partial; p.qkv_splits = qkv_splits; p.qkv_out = qkv_out; p.pos = pos;
      p.rope = rope; p.q_out = st->taps ? at<uint16_t>(ws, L.q) : nullptr; p.summary = ly->kv_summary;
      if ((rc = launch_attn_partial(Q_PARTIAL, L_DENSE, p, s)) != BC_OK) return rc;
    }
    if (!fold_reduce && (rc = launch_attn_reduce(r, s)) != BC_OK) return rc;
  }

  // S2 = top-k(a) (GEMV prologue); h1 = h + W_o a, left as chunk partials
  // for the gate|up prologue when it can form h1 itself
  const bool fold = gemv_sum_input_ok(m.d);
  int o_splits = 0;
  {
    ProjIn in{IN_SEL, a, nullptr, 0.f, nullptr, idx_o};
    if (fold_reduce) {
      in = ProjIn{IN_ATTN, nullptr, nullptr, 0.f, a, nullptr};
      in.am = at<float>(ws, L.m); in.al = at<float>(ws, L.l); in.ao = at<float>(ws, L.o);
      in.a_splits = n_splits; in.a_hd = hd;
    }
    FinishParams f{};
    f.y = h_mid; f.resid = hidden;
    if ((rc = run_gemv(ly->w_o, H * hd, m.d, k_d, in, partial2, fold ? FIN_NONE : FIN_RESID, f, s, &o_splits)) !=
        BC_OK)
      return rc;
  }

  // x2 = RMSNorm(h1), S3 (GEMV prologue); f = SiLU(gate) * up
  {
    const Pending h1{partial2, o_splits, hidden};
    const ProjIn in = norm_input(h_mid, fold ? &h1 : nullptr, h_mid, ly->g_mlp, eps, at<uint16_t>(ws, L.x2), idx_gu);
    FinishParams f{};
    f.y = hff; f.d_ff = m.d_ff;
    if ((rc = run_gemv(ly->w_gu, m.d, 2 * m.d_ff, k_d, in, partial, FIN_SWIGLU, f, s)) != BC_OK) return rc;
  }

  // S4 = top-k(f) (GEMV prologue); h = h1 + W_down f, stored or left pending
  {
    const ProjIn in{IN_SEL, hff, nullptr, 0.f, nullptr, idx_down};
    FinishParams f{};
    f.y = hidden; f.resid = h_mid;
    const bool defer = pout != nullptr && fold;
    int down_splits = 0;
    if ((rc = run_gemv(ly->w_down, m.d_ff, m.d, k_ff, in, partial2, defer ? FIN_NONE : FIN_RESID, f, s,
                       &down_splits)) != BC_OK)
      return rc;
    if (pout) *pout = defer ? Pending{partial2, down_splits, h_mid} : Pending{nullptr, 0, nullptr};
  }

  if (const bc_layer_taps* t = st->taps) {
    const size_t qb = size_t(H) * hd * 2;
    if ((rc = copy_tap(t->x1, at<void>(ws, L.x1), size_t(m.d) * 2, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_qkv, idx_qkv, size_t(k_d) * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->q, at<void>(ws, L.q), qb, s)) != BC_OK) return rc;
    for (int g = 0; g < Hkv && (t->k || t->v); ++g) {
      const size_t src = (size_t(g) * ly->n_cap + pos) * hd;
      if (t->k && (rc = copy_tap(t->k + size_t(g) * hd, ly->k_cache + src, size_t(hd) * 2, s)) != BC_OK) return rc;
      if (t->v && (rc = copy_tap(t->v + size_t(g) * hd, ly->v_cache + src, size_t(hd) * 2, s)) != BC_OK) return rc;
    }
    if (kv_sparse && (rc = copy_tap(t->idx_kv, at<void>(ws, L.idx_kv), size_t(Hkv) * n_sel * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->a, a, qb, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_o, idx_o, size_t(k_d) * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->h_mid, h_mid, size_t(m.d) * 2, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->x2, at<void>(ws, L.x2), size_t(m.d) * 2, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_gu, idx_gu, size_t(k_d) * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->hff, hff, size_t(m.d_ff) * 2, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_down, idx_down, size_t(k_ff) * 4, s)) != BC_OK) return rc;
    const size_t ml = masked ? 0 : size_t(H) * n_splits * 4;   // the masked baseline has no split partials
    if ((rc = copy_tap(t->attn_m, at<void>(ws, L.m), ml, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->attn_l, at<void>(ws, L.l), ml, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->attn_o, at<void>(ws, L.o), ml * hd, s)) != BC_OK) return rc;
  }
  return BC_OK;
}

// A step workspace: the layer layout, then the LM head's.
struct StepLayout { LayerLayout layer; HeadLayout head; size_t total; };
StepLayout step_layout(const bc_model_dims& m, int n_ctx, int n_splits) {
  StepLayout S;
  S.layer = layer_layout(m, n_ctx, n_splits);
  S.head = head_layout(m, S.layer.total);
  S.total = S.head.total;
  return S;
}

}  // namespace

extern "C" int bc_decode_layer(const bc_model_dims* dims, const bc_layer* ly, const bc_step* st, uint16_t* hidden,
                               void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != BC_OK) return rc;
  if (!ly || !st || !hidden || !ws) return set_error(BC_ERR_INVALID, "bc_decode_layer: NULL argument");
  if ((rc = check_layer(ly, st)) != BC_OK || (rc = check_step(st)) != BC_OK ||
      (rc = check_masked(*dims, ly, st)) != BC_OK)
    return rc;
  bc_kv_budget_info bud;
  if ((rc = bc_kv_budget(st->n_ctx, &st->kv, &bud)) != BC_OK) return rc;
  const int n_splits = step_splits(*dims, st, bud);
  const LayerLayout L = layer_layout(*dims, st->n_ctx, n_splits);
  if (ws_bytes < L.total) return set_error(BC_ERR_WORKSPACE, "bc_decode_layer: workspace %zu < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_error(BC_ERR_INVALID, "bc_decode_layer: ws not 256-byte aligned");
  return layer_body(*dims, ly, st, bud, n_splits, hidden, nullptr, nullptr, ws, L, static_cast<hipStream_t>(stream));
}

extern "C" size_t bc_step_workspace_bytes(const bc_model_dims* dims, int max_ctx, int max_splits) {
  if (check_dims(dims) != BC_OK || max_ctx < 1 || max_splits < 1 || dims->vocab <= 0) return 0;
  return step_layout(*dims, max_ctx, max_splits).total;
}

namespace {

// Arguments of a whole step, checked on the host; fills *S with the step's
// workspace layout.
int check_step_call(const bc_model_dims* dims, const bc_layer* layers, int n_layers, const uint16_t* g_final,
                    const uint16_t* w_head, const bc_step* st, uint16_t* hidden, float* logits, int32_t* token,
                    const char* who, bc_kv_budget_info* bud, int* n_splits, StepLayout* S) {
  int rc = check_dims(dims);
  if (rc != BC_OK) return rc;
  if (!layers || n_layers < 1 || !g_final || !w_head || !st || !hidden || !logits || !token)
    return set_error(BC_ERR_INVALID, "%s: NULL argument or no layers", who);
  if (dims->vocab <= 0 || dims->vocab % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "%s: vocab %% 8 != 0", who);
  if ((rc = check_step(st)) != BC_OK) return rc;
  for (int i = 0; i < n_layers; ++i)
    if ((rc = check_layer(&layers[i], st)) != BC_OK || (rc = check_masked(*dims, &layers[i], st)) != BC_OK) return rc;
  if ((rc = bc_kv_budget(st->n_ctx, &st->kv, bud)) != BC_OK) return rc;
  *n_splits = step_splits(*dims, st, *bud);
  *S = step_layout(*dims, st->n_ctx, *n_splits);
  return BC_OK;
}

int step_body(const bc_model_dims& m, const bc_layer* layers, int n_layers, const uint16_t* g_final,
              const uint16_t* w_head, const bc_step* st, const bc_kv_budget_info& bud, int n_splits,
              const StepLayout& S, uint16_t* hidden, float* logits, int32_t* token, void* ws, hipStream_t s) {
  int rc;
  bc_step one = *st;
  one.taps = nullptr;
  // each layer's output stays pending (down partials + h1) until the next
  // layer's q/k/v prologue, or the LM head's, forms and stores it
  Pending pend{nullptr, 0, nullptr};
  for (int i = 0; i < n_layers; ++i) {
    Pending next{nullptr, 0, nullptr};
    if ((rc = layer_body(m, &layers[i], &one, bud, n_splits, hidden, pend.partial ? &pend : nullptr, &next, ws,
                         S.layer, s)) != BC_OK)
      return rc;
    pend = next;
  }
  return run_head(m, hidden, pend.partial ? &pend : nullptr, g_final, w_head, float(st->rms_eps), logits, token,
                  at<float>(ws, S.head.partial), at<float>(ws, S.head.tile_max), at<int32_t>(ws, S.head.tile_arg), s);
}

}  // namespace

extern "C" int bc_decode_step(const bc_model_dims* dims, const bc_layer* layers, int n_layers, const uint16_t* g_final,
                              const uint16_t* w_head, const bc_step* st, uint16_t* hidden, float* logits,
                              int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  bc_kv_budget_info bud;
  int n_splits = 0;
  StepLayout S;
  int rc = check_step_call(dims, layers, n_layers, g_final, w_head, st, hidden, logits, token, "bc_decode_step",
                           &bud, &n_splits, &S);
  if (rc != BC_OK) return rc;
  if (!ws) return set_error(BC_ERR_INVALID, "bc_decode_step: NULL workspace");
  if (ws_bytes < S.total) return set_error(BC_ERR_WORKSPACE, "bc_decode_step: workspace %zu < %zu", ws_bytes, S.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_error(BC_ERR_INVALID, "bc_decode_step: ws not 256-byte aligned");
  return step_body(*dims, layers, n_layers, g_final, w_head, st, bud, n_splits, S, hidden, logits, token, ws,
                   static_cast<hipStream_t>(stream));
}

// ------------------------------------------------- allocation-free step
// The workspace of bc_decode_step_noalloc: one static device array, which
// every GPU the library runs on holds (at its own address) until the process
// ends.  Host code never uses the array's name as an address: the address is
// looked up once per device with hipGetSymbolAddress and kept in
// g_scratch_ptr, and only that pointer reaches kernels.
static __device__ __align__(256) unsigned char scratch[BC_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`.  The first call on a device (that
// device current) looks it up and enqueues one fill kernel on `s` that
// clears it.
int scratch_on_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(BC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(BC_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(BC_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    const int rc = launch_fill_zero(p, BC_STATIC_SCRATCH_BYTES, s);
    if (rc != BC_OK) return rc;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BC_OK;
}
}  // namespace

extern "C" int bc_decode_step_noalloc(const bc_model_dims* dims, const bc_layer* layers, int n_layers,
                                      const uint16_t* g_final, const uint16_t* w_head, const bc_step* st,
                                      uint16_t* hidden, float* logits, int32_t* token, void* stream) {
  bc_kv_budget_info bud;
  int n_splits = 0;
  StepLayout S;
  int rc = check_step_call(dims, layers, n_layers, g_final, w_head, st, hidden, logits, token,
                           "bc_decode_step_noalloc", &bud, &n_splits, &S);
  if (rc != BC_OK) return rc;
  if (S.total > size_t(BC_STATIC_SCRATCH_BYTES))
    return set_error(BC_ERR_WORKSPACE,
                     "bc_decode_step_noalloc: this step needs %zu bytes of workspace, above the static %u "
                     "(use bc_decode_step with a workspace)", S.total, unsigned(BC_STATIC_SCRATCH_BYTES));
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = scratch_on_device(s, &ws)) != BC_OK) return rc;
  return step_body(*dims, layers, n_layers, g_final, w_head, st, bud, n_splits, S, hidden, logits, token, ws, s);
}

// ------------------------------------------------------------------ LM head
extern "C" size_t bc_lm_head_workspace_bytes(const bc_model_dims* dims) {
  if (check_dims(dims) != BC_OK || dims->vocab <= 0 || dims->vocab % 8 != 0) return 0;
  return head_layout(*dims).total;
}

extern "C" int bc_lm_head(const bc_model_dims* dims, const uint16_t* hidden, const uint16_t* g_final,
                          const uint16_t* w_head_t, float* logits, int32_t* token, double rms_eps, void* ws,
                          size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != BC_OK) return rc;
  if (!hidden || !g_final || !w_head_t || !logits || !token || !ws)
    return set_error(BC_ERR_INVALID, "bc_lm_head: NULL pointer");
  if (dims->vocab <= 0 || dims->vocab % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "bc_lm_head: vocab %% 8 != 0");
  const HeadLayout L = head_layout(*dims);
  if (ws_bytes < L.total) return set_error(BC_ERR_WORKSPACE, "bc_lm_head: workspace %zu < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 15) return set_error(BC_ERR_INVALID, "bc_lm_head: ws not 16-byte aligned");
  return run_head(*dims, const_cast<uint16_t*>(hidden), nullptr, g_final, w_head_t, float(rms_eps), logits, token,
                  at<float>(ws, L.partial),
                  at<float>(ws, L.tile_max), at<int32_t>(ws, L.tile_arg), static_cast<hipStream_t>(stream));
}
