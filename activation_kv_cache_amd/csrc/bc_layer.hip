// bc_layer.hip -- one decoder layer of the decode step, the LM head, and the
// small entry points of libbc (errors, budgets, workspace, packing).
//
// bc_decode_layer enqueues, on one stream and with no host synchronisation:
//   1. k_norm_select     x1 = RMSNorm(h); S1 = top-k(x1)           (1 work-group)
//   2. k_gemv<QKV>       q,k,v over S1; rotary; append k,v; refresh the block summary
//   3. k_kv_score, k_kv_block_select  (r_kv < 1 only)
//   4. k_attn_partial    split-K partials over the list (or 0..n-1)
//   5. k_attn_reduce     merge; its last work-group selects S2 = top-k(a)
//   6. k_gemv<RESID>     h1 = h + W_o a over S2; tail: x2 = RMSNorm(h1), S3
//   7. k_gemv<SWIGLU>    f = SiLU(gate) * up over S3; tail: S4 = top-k(f)
//   8. k_gemv<RESID>     h = h1 + W_down f over S4
// Every launch size depends only on host-known scalars.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {
thread_local char g_err[512] = "";
constexpr int kOneGroupThreads = 1024;
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

namespace {

__global__ __launch_bounds__(kOneGroupThreads) void k_norm_select(const uint16_t* h, const uint16_t* g, int d,
                                                                 float eps, uint16_t* x_out, int k,
                                                                 int32_t* idx_out) {
  __shared__ TopkSmem<kOneGroupThreads> sm;
  __shared__ float part[kOneGroupThreads / kWave];
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int i = tid; i < d; i += kOneGroupThreads) {
    const float v = bf16_to_f32(h[i]);
    s += v * v;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
  if (wave_lane() == 0) part[tid >> 6] = s;
  __syncthreads();
  float ss = 0.f;
#pragma unroll
  for (int w = 0; w < kOneGroupThreads / kWave; ++w) ss += part[w];
  const float inv = 1.0f / sqrtf(ss / float(d) + eps);
  for (int i = tid; i < d; i += kOneGroupThreads)
    x_out[i] = f32_to_bf16(bf16_to_f32(h[i]) * inv * bf16_to_f32(g[i]));
  __syncthreads();
  if (idx_out == nullptr || k >= d) return;
  auto key = [x_out](int i) -> uint32_t { return uint32_t(x_out[i]) & 0x7FFFu; };
  auto emit = [idx_out](int r, int i) { idx_out[r] = i; };
  block_topk<kOneGroupThreads, 15>(d, k, key, emit, sm);
}

__global__ __launch_bounds__(kOneGroupThreads) void k_select(const uint16_t* x, int n, int k, int32_t* idx_out) {
  __shared__ TopkSmem<kOneGroupThreads> sm;
  auto key = [x](int i) -> uint32_t { return uint32_t(x[i]) & 0x7FFFu; };
  auto emit = [idx_out](int r, int i) { idx_out[r] = i; };
  block_topk<kOneGroupThreads, 15>(n, k, key, emit, sm);
}

__global__ void k_fill_zero(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0)
    for (size_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

__global__ __launch_bounds__(256) void k_pack_gate_up(const uint16_t* gate, const uint16_t* up, int d_ff,
                                                     uint16_t* out) {
  const size_t row = blockIdx.x;
  const uint16_t* gr = gate + row * d_ff;
  const uint16_t* ur = up + row * d_ff;
  uint16_t* orow = out + row * size_t(2) * d_ff;
  for (int c = threadIdx.x; c < 2 * d_ff; c += 256) {
    const int t = c / kGemvTile, off = c % kGemvTile;
    const int w = min(kGemvTile / 2, d_ff - t * (kGemvTile / 2));
    orow[c] = off < w ? gr[t * (kGemvTile / 2) + off] : ur[t * (kGemvTile / 2) + off - w];
  }
}

// ------------------------------------------------------------ layer layout
struct LayerLayout {
  size_t counters, partial, x1, idx_qkv, q, scores, idx_kv, m, l, o, a, idx_o, h_mid, x2, idx_gu, hff, idx_down;
  size_t total;
};
constexpr int kCounterSlots = 5;      // qkv, o, gate|up, down, attention merge
constexpr int kCounterWords = 1024;

size_t gemv_partial_max(const bc_model_dims& m) {
  const int qkv = m.n_heads * m.head_dim + 2 * m.n_kv_heads * m.head_dim;
  size_t mx = 0;
  const int outs[4] = {qkv, m.d, 2 * m.d_ff, m.d};
  const int ins[4] = {m.d, m.n_heads * m.head_dim, m.d, m.d_ff};
  for (int i = 0; i < 4; ++i) {
    GemvPlan pl = plan_gemv(outs[i], ins[i]);
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
  L.counters = take(size_t(kCounterSlots) * kCounterWords * 4);
  L.partial = take(gemv_partial_max(m));
  L.x1 = take(size_t(m.d) * 2);
  L.idx_qkv = take(size_t(m.d) * 4);
  L.q = take(size_t(H) * hd * 2);
  L.scores = take(size_t(Hkv) * nb * 4);
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
  if (m->d > 65536 || m->d_ff > 65536) return set_error(BC_ERR_UNSUPPORTED, "dims: d, d_ff <= 65536");
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

int launch_norm_select(const uint16_t* h, const uint16_t* g, int d, float eps, uint16_t* x_out, int k,
                       int32_t* idx_out, hipStream_t s) {
  k_norm_select<<<1, kOneGroupThreads, 0, s>>>(h, g, d, eps, x_out, k, idx_out);
  return check_launch("k_norm_select");
}

int launch_select(const uint16_t* x, int n, int k, int32_t* idx_out, hipStream_t s) {
  k_select<<<1, kOneGroupThreads, 0, s>>>(x, n, k, idx_out);
  return check_launch("k_select");
}

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
  k_pack_gate_up<<<dim3(d), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(w_gate_t, w_up_t, d_ff, w_gu);
  return check_launch("k_pack_gate_up");
}

extern "C" size_t bc_layer_workspace_bytes(const bc_model_dims* dims, int max_ctx, int max_splits) {
  if (check_dims(dims) != BC_OK || max_ctx < 1 || max_splits < 1) return 0;
  return layer_layout(*dims, max_ctx, max_splits).total;
}

extern "C" int bc_decode_layer(const bc_model_dims* dims, const bc_layer* ly, const bc_step* st, uint16_t* hidden,
                               void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != BC_OK) return rc;
  if (!ly || !st || !hidden || !ws) return set_error(BC_ERR_INVALID, "bc_decode_layer: NULL argument");
  if (!ly->w_qkv || !ly->w_o || !ly->w_gu || !ly->w_down || !ly->g_attn || !ly->g_mlp || !ly->k_cache ||
      !ly->v_cache)
    return set_error(BC_ERR_INVALID, "bc_decode_layer: NULL layer pointer");
  if (ly->n_cap <= 0 || ly->n_cap % 16 != 0) return set_error(BC_ERR_INVALID, "bc_decode_layer: n_cap %% 16 != 0");
  if (st->n_ctx < 1 || st->n_ctx > ly->n_cap)
    return set_error(BC_ERR_INVALID, "bc_decode_layer: n_ctx=%d outside [1, n_cap=%d]", st->n_ctx, ly->n_cap);
  if (!(st->r_p > 0.0)) return set_error(BC_ERR_INVALID, "bc_decode_layer: r_p must be > 0");
  if (!(st->rms_eps >= 0.0) || !(st->rope_theta > 0.0)) return set_error(BC_ERR_INVALID, "bc_decode_layer: eps/theta");
  const bool kv_sparse = st->kv.r_kv < 1.0;
  if (kv_sparse && !ly->kv_summary) return set_error(BC_ERR_INVALID, "bc_decode_layer: r_kv < 1 needs kv_summary");
  bc_kv_budget_info bud;
  rc = bc_kv_budget(st->n_ctx, &st->kv, &bud);
  if (rc != BC_OK) return rc;
  const bc_model_dims& m = *dims;
  const int hd = m.head_dim, H = m.n_heads, Hkv = m.n_kv_heads;
  const int n_sel = kv_sparse ? bud.t_sel : st->n_ctx;
  int n_splits = st->n_splits > 0 ? st->n_splits : bc_attn_default_splits(n_sel, Hkv);
  if (n_splits > 4096) return set_error(BC_ERR_INVALID, "bc_decode_layer: n_splits=%d", n_splits);
  const LayerLayout L = layer_layout(m, st->n_ctx, n_splits);
  if (ws_bytes < L.total) return set_error(BC_ERR_WORKSPACE, "bc_decode_layer: workspace %zu < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_error(BC_ERR_INVALID, "bc_decode_layer: ws not 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool sparse = st->r_p < 1.0;
  const int k_d = bc_channel_keep(st->r_p, m.d);
  const int k_ff = bc_channel_keep(st->r_p, m.d_ff);
  const int qkv_out = H * hd + 2 * Hkv * hd;
  const int pos = st->n_ctx - 1;
  uint32_t* counters = at<uint32_t>(ws, L.counters);
  float* partial = at<float>(ws, L.partial);
  const float eps = float(st->rms_eps);

  // 1. x1 = RMSNorm(h), S1
  rc = launch_norm_select(hidden, ly->g_attn, m.d, eps, at<uint16_t>(ws, L.x1), k_d,
                          sparse ? at<int32_t>(ws, L.idx_qkv) : nullptr, s);
  if (rc != BC_OK) return rc;

  // 2. q, k, v; rotary; append; summary
  {
    GemvPlan pl = plan_gemv(qkv_out, k_d);
    GemvParams p{};
    p.wt = ly->w_qkv; p.d_in = m.d; p.d_out = qkv_out; p.x = at<uint16_t>(ws, L.x1);
    p.idx = sparse ? at<int32_t>(ws, L.idx_qkv) : nullptr; p.k = k_d;
    p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
    p.partial = partial; p.counters = counters + 0 * kCounterWords;
    p.q_out = at<uint16_t>(ws, L.q); p.k_cache = ly->k_cache; p.v_cache = ly->v_cache;
    p.summary = ly->kv_summary;
    p.n_heads = H; p.n_kv_heads = Hkv; p.head_dim = hd; p.n_cap = ly->n_cap; p.pos = pos;
    p.theta = st->rope_theta;
    p.tail = TAIL_NONE;
    if ((rc = launch_gemv(EPI_QKV, p, s)) != BC_OK) return rc;
  }

  // 3. KV selection
  if (kv_sparse) {
    KvSelectParams p{};
    p.q = at<uint16_t>(ws, L.q); p.summary = ly->kv_summary; p.nb_cap = ly->n_cap / 16; p.n_ctx = st->n_ctx;
    p.n_heads = H; p.n_kv_heads = Hkv; p.head_dim = hd; p.bud = bud;
    p.scores = at<float>(ws, L.scores); p.idx_out = at<int32_t>(ws, L.idx_kv);
    if ((rc = launch_kv_score_select(p, s)) != BC_OK) return rc;
  }

  // 4-5. attention; S2 = top-k(a)
  {
    AttnParams p{};
    p.q = at<uint16_t>(ws, L.q); p.k_cache = ly->k_cache; p.v_cache = ly->v_cache; p.n_cap = ly->n_cap;
    p.idx = kv_sparse ? at<int32_t>(ws, L.idx_kv) : nullptr; p.n_sel = n_sel;
    p.n_heads = H; p.n_kv_heads = Hkv; p.head_dim = hd; p.n_splits = n_splits;
    p.scale_log2 = float(1.4426950408889634 / sqrt(double(hd)));
    p.m = at<float>(ws, L.m); p.l = at<float>(ws, L.l); p.o = at<float>(ws, L.o);
    if ((rc = launch_attn_partial(p, s)) != BC_OK) return rc;
    ReduceParams r{};
    r.m = p.m; r.l = p.l; r.o = p.o; r.n_heads = H; r.n_splits = n_splits; r.head_dim = hd;
    r.out = at<uint16_t>(ws, L.a);
    r.counters = sparse ? counters + 4 * kCounterWords : nullptr;
    r.tail_k = k_d; r.tail_idx_out = at<int32_t>(ws, L.idx_o);
    if ((rc = launch_attn_reduce(r, s)) != BC_OK) return rc;
  }

  // 6. h1 = h + W_o a; tail: x2 = RMSNorm(h1), S3
  {
    GemvPlan pl = plan_gemv(m.d, k_d);
    GemvParams p{};
    p.wt = ly->w_o; p.d_in = H * hd; p.d_out = m.d; p.x = at<uint16_t>(ws, L.a);
    p.idx = sparse ? at<int32_t>(ws, L.idx_o) : nullptr; p.k = k_d;
    p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
    p.partial = partial; p.counters = counters + 1 * kCounterWords;
    p.y = at<uint16_t>(ws, L.h_mid); p.resid = hidden;
    p.tail = TAIL_NORM_SELECT; p.tail_in = at<uint16_t>(ws, L.h_mid); p.tail_n = m.d; p.tail_gain = ly->g_mlp;
    p.tail_eps = eps; p.tail_x_out = at<uint16_t>(ws, L.x2); p.tail_k = sparse ? k_d : m.d;
    p.tail_idx_out = at<int32_t>(ws, L.idx_gu);
    if ((rc = launch_gemv(EPI_RESID, p, s)) != BC_OK) return rc;
  }

  // 7. f = SiLU(gate) * up; tail: S4
  {
    GemvPlan pl = plan_gemv(2 * m.d_ff, k_d);
    GemvParams p{};
    p.wt = ly->w_gu; p.d_in = m.d; p.d_out = 2 * m.d_ff; p.x = at<uint16_t>(ws, L.x2);
    p.idx = sparse ? at<int32_t>(ws, L.idx_gu) : nullptr; p.k = k_d;
    p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
    p.partial = partial; p.counters = counters + 2 * kCounterWords;
    p.y = at<uint16_t>(ws, L.hff); p.d_ff = m.d_ff;
    if (sparse) {
      p.tail = TAIL_SELECT; p.tail_in = at<uint16_t>(ws, L.hff); p.tail_n = m.d_ff; p.tail_k = k_ff;
      p.tail_idx_out = at<int32_t>(ws, L.idx_down);
    } else {
      p.tail = TAIL_NONE;
    }
    if ((rc = launch_gemv(EPI_SWIGLU, p, s)) != BC_OK) return rc;
  }

  // 8. h = h1 + W_down f
  {
    GemvPlan pl = plan_gemv(m.d, k_ff);
    GemvParams p{};
    p.wt = ly->w_down; p.d_in = m.d_ff; p.d_out = m.d; p.x = at<uint16_t>(ws, L.hff);
    p.idx = sparse ? at<int32_t>(ws, L.idx_down) : nullptr; p.k = k_ff;
    p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
    p.partial = partial; p.counters = counters + 3 * kCounterWords;
    p.y = hidden; p.resid = at<uint16_t>(ws, L.h_mid);
    p.tail = TAIL_NONE;
    if ((rc = launch_gemv(EPI_RESID, p, s)) != BC_OK) return rc;
  }

  if (const bc_layer_taps* t = st->taps) {
    const size_t qb = size_t(H) * hd * 2, kvb = size_t(Hkv) * hd * 2;
    if ((rc = copy_tap(t->x1, at<void>(ws, L.x1), size_t(m.d) * 2, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_qkv, at<void>(ws, L.idx_qkv), size_t(k_d) * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->q, at<void>(ws, L.q), qb, s)) != BC_OK) return rc;
    for (int g = 0; g < Hkv && (t->k || t->v); ++g) {
      const size_t src = (size_t(g) * ly->n_cap + pos) * hd;
      if (t->k && (rc = copy_tap(t->k + size_t(g) * hd, ly->k_cache + src, size_t(hd) * 2, s)) != BC_OK) return rc;
      if (t->v && (rc = copy_tap(t->v + size_t(g) * hd, ly->v_cache + src, size_t(hd) * 2, s)) != BC_OK) return rc;
    }
    (void)kvb;
    if (kv_sparse && (rc = copy_tap(t->idx_kv, at<void>(ws, L.idx_kv), size_t(Hkv) * n_sel * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->a, at<void>(ws, L.a), qb, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_o, at<void>(ws, L.idx_o), size_t(k_d) * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->h_mid, at<void>(ws, L.h_mid), size_t(m.d) * 2, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->x2, at<void>(ws, L.x2), size_t(m.d) * 2, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_gu, at<void>(ws, L.idx_gu), size_t(k_d) * 4, s)) != BC_OK) return rc;
    if ((rc = copy_tap(t->hff, at<void>(ws, L.hff), size_t(m.d_ff) * 2, s)) != BC_OK) return rc;
    if (sparse && (rc = copy_tap(t->idx_down, at<void>(ws, L.idx_down), size_t(k_ff) * 4, s)) != BC_OK) return rc;
  }
  return BC_OK;
}

// ------------------------------------------------------------------ LM head
namespace {
struct HeadLayout { size_t counters, partial, x, tile_max, tile_arg, total; };
HeadLayout head_layout(const bc_model_dims& m) {
  GemvPlan pl = plan_gemv(m.vocab, m.d);
  HeadLayout L;
  size_t off = 0;
  auto take = [&off](size_t bytes) { size_t o = off; off += align_up(bytes > 0 ? bytes : 1, 256); return o; };
  L.counters = take(pl.counter_bytes);
  L.partial = take(pl.partial_bytes);
  L.x = take(size_t(m.d) * 2);
  L.tile_max = take(size_t(pl.n_tiles) * 4);
  L.tile_arg = take(size_t(pl.n_tiles) * 4);
  L.total = off;
  return L;
}
}  // namespace

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
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_norm_select(hidden, g_final, dims->d, float(rms_eps), at<uint16_t>(ws, L.x), dims->d, nullptr, s);
  if (rc != BC_OK) return rc;
  GemvPlan pl = plan_gemv(dims->vocab, dims->d);
  GemvParams p{};
  p.wt = w_head_t; p.d_in = dims->d; p.d_out = dims->vocab; p.x = at<uint16_t>(ws, L.x); p.idx = nullptr;
  p.k = dims->d; p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
  p.partial = at<float>(ws, L.partial); p.counters = at<uint32_t>(ws, L.counters);
  p.yf = logits; p.tile_max = at<float>(ws, L.tile_max); p.tile_arg = at<int32_t>(ws, L.tile_arg);
  p.token_out = token; p.tail = TAIL_ARGMAX;
  return launch_gemv(EPI_F32_ARGMAX, p, s);
}
