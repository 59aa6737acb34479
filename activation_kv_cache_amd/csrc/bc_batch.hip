// bc_batch.hip -- one decoder layer (and a whole step) for a batch of up to
// four sequences that share the weights, for gfx950.
//
// README "Quick start" / "Usage", the byte account of crossover_batch: a
// batch reads the projection weights once for the union of the channels its
// sequences keep, and pays the key-value bytes once per sequence.  Every
// sequence keeps its own exact top-k channels and gets exactly its own
// sparse GEMV (bc_sparse_gemv_batch reads the union's rows once); its
// cache, block summaries, norms, rotary, KV selection and attention are its
// own.  All sequences of a call attend to the same number of tokens.
//
// Per layer, on one stream:
//   k_batch_norm            x1_b = RMSNorm(h_b) * g_attn            (one work-group per sequence)
//   k_select_reg (grid b)   S1_b = top-k(|x1_b|)                     (r_p < 1)
//   k_gemv_batch            [q k v]_b over the union of the S1_b     (fp32)
//   k_batch_rope_append     rotary on q_b, k_b; k_b, v_b written at slot n-1 of sequence b's cache; that
//                           block's (min, max) summary refreshed
//   per sequence            KV list (r_kv < 1: scores + list), split-K attention, merge -> a_b
//   k_select_reg, k_gemv_batch   S2_b = top-k(|a_b|); o_b
//   k_batch_norm            h1_b = bf16(h_b + o_b); x2_b = RMSNorm(h1_b) * g_mlp
//   k_select_reg, k_gemv_batch   S3_b; [gate | up]_b (fp32, tile-interleaved columns)
//   k_batch_swiglu          f_b = SiLU(gate_b) * up_b
//   k_select_reg, k_gemv_batch   S4_b = top-k(|f_b|); down_b
//   k_batch_resid           h_b = bf16(h1_b + down_b)
// The projection outputs pass between these kernels in fp32, so every
// value is rounded where the single-sequence layer rounds it; the sums over
// the kept channels are added in another order (the union GEMV's ranges).
#include <math.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

constexpr int kBatchThreads = 1024;
constexpr int kBatchSeqMax = 4;

struct BatchNormParams {
  const uint16_t* h;      // [batch][d]
  const float* add;       // optional [batch][add_stride] fp32: h_b = bf16(h_b + add_b) first
  int add_stride;
  uint16_t* h_out;        // with add: the sum, [batch][d]
  const uint16_t* gain;   // [d]
  int d;
  float eps;
  uint16_t* x_out;        // [batch][d]
};

// x = bf16(RMSNorm(h) * gain) of sequence blockIdx.x, with the sum of
// squares in the fixed order of the GEMV prologue (the thread's channels in
// order, the wave tree, the waves in order).
__global__ __launch_bounds__(kBatchThreads) void k_batch_norm(const BatchNormParams p) {
  __shared__ float part[kBatchThreads / kWave];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int PM = 16;   // channels per thread (d <= 16384)
  const int P = (p.d + kBatchThreads - 1) / kBatchThreads;
  const int c0 = tid * P;
  float v[PM];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < PM; ++e) {
    const int c = c0 + e;
    float x = 0.f;
    if (e < P && c < p.d) {
      x = bf16_to_f32(p.h[size_t(b) * p.d + c]);
      if (p.add) {
        x = bf16_to_f32(f32_to_bf16(p.add[size_t(b) * p.add_stride + c] + x));
        p.h_out[size_t(b) * p.d + c] = f32_to_bf16(x);
      }
    }
    v[e] = x;
    ss += x * x;
  }
  ss = wave_sum_f32(ss);
  if (lane == 0) part[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int ww = 0; ww < kBatchThreads / kWave; ++ww) tot += part[ww];
  const float inv = 1.0f / sqrtf(tot / float(p.d) + p.eps);
#pragma unroll
  for (int e = 0; e < PM; ++e) {
    const int c = c0 + e;
    if (e < P && c < p.d) p.x_out[size_t(b) * p.d + c] = f32_to_bf16(v[e] * inv * bf16_to_f32(p.gain[c]));
  }
}

struct RopeAppendParams {
  const float* y;         // [batch][qkv_out]: q | k | v (fp32)
  int qkv_out, n_heads, n_kv_heads, head_dim, n_cap, pos;
  RopeTable rope;
  uint16_t* q_out;        // [batch][n_heads][head_dim]
  uint16_t* k_cache[kBatchSeqMax];
  uint16_t* v_cache[kBatchSeqMax];
  uint16_t* summary[kBatchSeqMax];   // may be NULL
};

// grid (n_heads + n_kv_heads, batch), head_dim / 2 threads: thread i turns
// the pair (i, i + D/2) of one q or k head; the k heads' threads also store
// v and refresh the block summary of their two dims.
__global__ __launch_bounds__(64) void k_batch_rope_append(const RopeAppendParams p) {
  const int hh = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int D = p.head_dim, half = D / 2;
  if (i >= half) return;
  const float* yb = p.y + size_t(b) * p.qkv_out;
  const float c = p.rope.c[i], s = p.rope.s[i];
  if (hh < p.n_heads) {
    const float a = yb[hh * D + i], bb = yb[hh * D + i + half];
    uint16_t* q = p.q_out + (size_t(b) * p.n_heads + hh) * D;
    q[i] = f32_to_bf16(a * c - bb * s);
    q[i + half] = f32_to_bf16(bb * c + a * s);
    return;
  }
  const int g = hh - p.n_heads;
  const int kb = p.n_heads * D + g * D, vb = p.n_heads * D + p.n_kv_heads * D + g * D;
  const float a = yb[kb + i], bb = yb[kb + i + half];
  const uint16_t k0 = f32_to_bf16(a * c - bb * s), k1 = f32_to_bf16(bb * c + a * s);
  uint16_t* K = p.k_cache[b] + (size_t(g) * p.n_cap) * D;
  uint16_t* V = p.v_cache[b] + (size_t(g) * p.n_cap) * D;
  K[size_t(p.pos) * D + i] = k0;
  K[size_t(p.pos) * D + i + half] = k1;
  V[size_t(p.pos) * D + i] = f32_to_bf16(yb[vb + i]);
  V[size_t(p.pos) * D + i + half] = f32_to_bf16(yb[vb + i + half]);
  if (p.summary[b]) {
    // (min, max) over the block's tokens up to pos, in token order: the
    // first of equal values is kept (+0 and -0 as the block summary build)
    const int blk = p.pos / 16;
    float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
    uint16_t bmn0 = 0, bmx0 = 0, bmn1 = 0, bmx1 = 0;
    for (int t = 16 * blk; t <= p.pos; ++t) {
      const uint16_t u0 = t == p.pos ? k0 : K[size_t(t) * D + i];
      const uint16_t u1 = t == p.pos ? k1 : K[size_t(t) * D + i + half];
      const float f0 = bf16_to_f32(u0), f1 = bf16_to_f32(u1);
      if (f0 < mn0) { mn0 = f0; bmn0 = u0; }
      if (f0 > mx0) { mx0 = f0; bmx0 = u0; }
      if (f1 < mn1) { mn1 = f1; bmn1 = u1; }
      if (f1 > mx1) { mx1 = f1; bmx1 = u1; }
    }
    uint16_t* sm = p.summary[b] + ((size_t(g) * (p.n_cap / 16) + blk) * D) * 2;
    sm[2 * i] = bmn0;
    sm[2 * i + 1] = bmx0;
    sm[2 * (i + half)] = bmn1;
    sm[2 * (i + half) + 1] = bmx1;
  }
}

// f_b = bf16(SiLU(gate) * up) from the gate|up GEMV's fp32 output in the
// tile-interleaved column order of bc_pack_gate_up.
__global__ __launch_bounds__(256) void k_batch_swiglu(const float* y, int d_ff, uint16_t* f) {
  const int b = blockIdx.y;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= d_ff) return;
  const int t = u / (kGemvTile / 2), i = u % (kGemvTile / 2);
  const int w = min(kGemvTile / 2, d_ff - t * (kGemvTile / 2));
  const float* yb = y + size_t(b) * 2 * d_ff + size_t(t) * kGemvTile;
  const float g = yb[i], up = yb[w + i];
  f[size_t(b) * d_ff + u] = f32_to_bf16(g / (1.0f + expf(-g)) * up);
}

// h_b = bf16(y_b + h1_b), the single-sequence layer's residual arithmetic
__global__ __launch_bounds__(256) void k_batch_resid(const uint16_t* h1, const float* y, int n, uint16_t* h) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) h[i] = f32_to_bf16(y[i] + bf16_to_f32(h1[i]));
}

// Argmax of each sequence's fp32 logits (lowest index among equal maxima).
__global__ __launch_bounds__(1024) void k_batch_argmax(const float* logits, int vocab, int32_t* token) {
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int b = blockIdx.x, tid = threadIdx.x;
  float best = -INFINITY;
  int besti = 0x7FFFFFFF;
  for (int i = tid; i < vocab; i += 1024) {
    const float v = logits[size_t(b) * vocab + i];
    if (v > best) { best = v; besti = i; }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off, kWave);
    const int oi = __shfl_xor(besti, off, kWave);
    if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
  }
  if ((tid & 63) == 0) { bv[tid >> 6] = best; bi[tid >> 6] = besti; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w)
      if (bv[w] > best || (bv[w] == best && bi[w] < besti)) { best = bv[w]; besti = bi[w]; }
    token[b] = besti;
  }
}

}  // namespace
}  // namespace bc

namespace bc {
namespace {

struct BatchLayout {
  size_t x1, a, x2, f, i1, io, igu, idn, yq, yo, ygu, ydn, q, hmid, m, l, o, idx_kv, scores, gws, total;
};

BatchLayout batch_layout(const bc_model_dims& m, int B, int n_ctx, int n_splits) {
  BatchLayout L;
  size_t off = 0;
  auto take = [&off](size_t bytes) { size_t o = off; off += align_up(bytes > 0 ? bytes : 1, 256); return o; };
  const int H = m.n_heads, Hkv = m.n_kv_heads, hd = m.head_dim, d = m.d, dff = m.d_ff;
  const int qkv = H * hd + 2 * Hkv * hd;
  L.x1 = take(size_t(B) * d * 2);
  L.a = take(size_t(B) * H * hd * 2);
  L.x2 = take(size_t(B) * d * 2);
  L.f = take(size_t(B) * dff * 2);
  L.i1 = take(size_t(B) * d * 4);
  L.io = take(size_t(B) * H * hd * 4);
  L.igu = take(size_t(B) * d * 4);
  L.idn = take(size_t(B) * dff * 4);
  L.yq = take(size_t(B) * qkv * 4);
  L.yo = take(size_t(B) * d * 4);
  L.ygu = take(size_t(B) * 2 * dff * 4);
  L.ydn = take(size_t(B) * d * 4);
  L.q = take(size_t(B) * H * hd * 2);
  L.hmid = take(size_t(B) * d * 2);
  L.m = take(size_t(H) * n_splits * 4);
  L.l = take(size_t(H) * n_splits * 4);
  L.o = take(size_t(H) * n_splits * hd * 4);
  L.idx_kv = take(size_t(B) * Hkv * n_ctx * 4);
  L.scores = take(size_t(Hkv) * ((n_ctx + 15) / 16 + 1) * 4);
  size_t g = 0;
  const int ins[4] = {d, H * hd, d, dff}, outs[4] = {qkv, d, 2 * dff, d};
  for (int i = 0; i < 4; ++i) {
    const size_t b = bc_sparse_gemv_batch_workspace_bytes(ins[i], outs[i], ins[i], B);
    if (b > g) g = b;
  }
  const size_t hb = bc_sparse_gemv_batch_workspace_bytes(d, m.vocab > 0 ? m.vocab : 8, d, B);
  if (hb > g) g = hb;
  L.gws = take(g);
  L.total = off;
  return L;
}

template <typename T>
T* at_(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int check_batch_dims(const bc_model_dims* m) {
  if (m->d <= 0 || m->d_ff <= 0 || m->n_heads <= 0 || m->n_kv_heads <= 0 || m->head_dim <= 0)
    return set_error(BC_ERR_INVALID, "dims: non-positive size");
  if (m->n_heads * m->head_dim != m->d) return set_error(BC_ERR_INVALID, "dims: n_heads*head_dim != d");
  if (m->n_heads % m->n_kv_heads != 0) return set_error(BC_ERR_INVALID, "dims: n_heads %% n_kv_heads != 0");
  if (!valid_head_dim(m->head_dim)) return set_error(BC_ERR_UNSUPPORTED, "dims: head_dim %d", m->head_dim);
  if (!valid_group(m->n_heads / m->n_kv_heads)) return set_error(BC_ERR_UNSUPPORTED, "dims: group size");
  if (m->d % 8 != 0 || m->d_ff % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "dims: d and d_ff must be multiples of 8");
  return BC_OK;
}

int copy_tap_b(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (!dst || bytes == 0) return BC_OK;
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? BC_OK : set_error(BC_ERR_HIP, "tap copy: %s", hipGetErrorString(e));
}

// One batched projection: per-sequence top-k of x (when sparse) and the
// union GEMV; y fp32 [B][d_out].
int batch_proj(const uint16_t* wt, int d_in, int d_out, const uint16_t* x, int k, int B, int32_t* idx, float* y,
               void* gws, size_t gws_bytes, hipStream_t s) {
  int rc;
  const bool sparse = k < d_in;
  if (sparse && (rc = launch_select_batch(x, d_in, k, idx, B, d_in, s)) != BC_OK) return rc;
  return run_gemv_batch(wt, 1, d_in, d_out, x, sparse ? idx : nullptr, k, B, nullptr, y, nullptr, gws, gws_bytes, s);
}

int check_batch_layers(const bc_model_dims& m, const bc_layer* ly, int B, const bc_step* st) {
  if (B < 1 || B > kBatchSeqMax) return set_error(BC_ERR_UNSUPPORTED, "batch %d outside [1, %d]", B, kBatchSeqMax);
  if (st->masked_ws) return set_error(BC_ERR_UNSUPPORTED, "the batched layer has no masked-attention baseline");
  if (st->n_splits < 0 || st->n_splits > 4096) return set_error(BC_ERR_INVALID, "n_splits=%d", st->n_splits);
  if (!(st->r_p > 0.0)) return set_error(BC_ERR_INVALID, "r_p must be > 0");
  if (m.d > 16384 || m.d_ff > 16384) return set_error(BC_ERR_UNSUPPORTED, "batched GEMV inputs above 16384");
  for (int b = 0; b < B; ++b) {
    const bc_layer& l = ly[b];
    if (!l.w_qkv || !l.w_o || !l.w_gu || !l.w_down || !l.g_attn || !l.g_mlp || !l.k_cache || !l.v_cache)
      return set_error(BC_ERR_INVALID, "NULL layer pointer (sequence %d)", b);
    if (l.w_qkv != ly[0].w_qkv || l.w_o != ly[0].w_o || l.w_gu != ly[0].w_gu || l.w_down != ly[0].w_down ||
        l.g_attn != ly[0].g_attn || l.g_mlp != ly[0].g_mlp)
      return set_error(BC_ERR_INVALID, "sequence %d does not share the batch's weights", b);
    if (l.n_cap != ly[0].n_cap || l.n_cap <= 0 || l.n_cap % 16 != 0)
      return set_error(BC_ERR_INVALID, "n_cap must be equal, positive and a multiple of 16");
    if (st->n_ctx < 1 || st->n_ctx > l.n_cap) return set_error(BC_ERR_INVALID, "n_ctx=%d n_cap=%d", st->n_ctx, l.n_cap);
    if (st->kv.r_kv < 1.0 && !l.kv_summary) return set_error(BC_ERR_INVALID, "r_kv < 1 needs kv_summary");
  }
  return BC_OK;
}

// One batched layer.  hidden [B][d] in and out.
int batch_layer_body(const bc_model_dims& m, const bc_layer* ly, int B, const bc_step* st,
                     const bc_kv_budget_info& bud, int n_splits, uint16_t* hidden, const bc_layer_taps* taps,
                     void* ws, const BatchLayout& L, hipStream_t s) {
  int rc;
  const int H = m.n_heads, Hkv = m.n_kv_heads, hd = m.head_dim, d = m.d, dff = m.d_ff;
  const int qkv = H * hd + 2 * Hkv * hd;
  const int k_d = bc_channel_keep(st->r_p, d), k_ff = bc_channel_keep(st->r_p, dff);
  const bool kv_sparse = st->kv.r_kv < 1.0;
  const int n_sel = kv_sparse ? bud.t_sel : st->n_ctx;
  const float eps = float(st->rms_eps);
  void* gws = at_<void>(ws, L.gws);
  const size_t gws_bytes = L.total - L.gws;
  uint16_t *x1 = at_<uint16_t>(ws, L.x1), *a = at_<uint16_t>(ws, L.a), *x2 = at_<uint16_t>(ws, L.x2);
  uint16_t *f = at_<uint16_t>(ws, L.f), *q = at_<uint16_t>(ws, L.q), *hmid = at_<uint16_t>(ws, L.hmid);
  float *yq = at_<float>(ws, L.yq), *yo = at_<float>(ws, L.yo), *ygu = at_<float>(ws, L.ygu);
  float* ydn = at_<float>(ws, L.ydn);

  // x1 = RMSNorm(h); S1; q, k, v over the union
  BatchNormParams np{};
  np.h = hidden; np.gain = ly[0].g_attn; np.d = d; np.eps = eps; np.x_out = x1;
  k_batch_norm<<<dim3(B), dim3(kBatchThreads), 0, s>>>(np);
  if ((rc = check_launch("k_batch_norm")) != BC_OK) return rc;
  if ((rc = batch_proj(ly[0].w_qkv, d, qkv, x1, k_d, B, at_<int32_t>(ws, L.i1), yq, gws, gws_bytes, s)) !=
      BC_OK)
    return rc;
  RopeAppendParams rp{};
  rp.y = yq; rp.qkv_out = qkv; rp.n_heads = H; rp.n_kv_heads = Hkv; rp.head_dim = hd; rp.n_cap = ly[0].n_cap;
  rp.pos = st->n_ctx - 1; rp.q_out = q;
  rope_table(rp.pos, st->rope_theta, hd, &rp.rope);
  for (int b = 0; b < B; ++b) {
    rp.k_cache[b] = ly[b].k_cache; rp.v_cache[b] = ly[b].v_cache; rp.summary[b] = ly[b].kv_summary;
  }
  k_batch_rope_append<<<dim3(H + Hkv, B), dim3(64), 0, s>>>(rp);
  if ((rc = check_launch("k_batch_rope_append")) != BC_OK) return rc;

  // attention, one sequence after another (each reads its own cache)
  for (int b = 0; b < B; ++b) {
    const uint16_t* qb = q + size_t(b) * H * hd;
    int32_t* idxb = at_<int32_t>(ws, L.idx_kv) + size_t(b) * Hkv * n_sel;
    if (kv_sparse) {
      KvSelectParams kp{};
      kp.q = qb; kp.summary = ly[b].kv_summary; kp.nb_cap = ly[b].n_cap / 16; kp.n_ctx = st->n_ctx;
      kp.n_heads = H; kp.n_kv_heads = Hkv; kp.head_dim = hd; kp.bud = bud;
      kp.scores = at_<float>(ws, L.scores); kp.scores_stride = bud.n_cand > 0 ? bud.n_cand : 1; kp.idx_out = idxb;
      if ((rc = launch_kv_score_select(kp, s)) != BC_OK) return rc;
    }
    AttnParams p{};
    p.q = qb; p.k_cache = ly[b].k_cache; p.v_cache = ly[b].v_cache; p.n_cap = ly[b].n_cap;
    p.n_sel = n_sel; p.n_heads = H; p.n_kv_heads = Hkv; p.head_dim = hd; p.n_splits = n_splits;
    p.scale_log2 = float(1.0 / sqrt(double(hd))) * 1.4426950408889634f;
    p.m = at_<float>(ws, L.m); p.l = at_<float>(ws, L.l); p.o = at_<float>(ws, L.o);
    p.idx = kv_sparse ? idxb : nullptr;
    if ((rc = launch_attn_partial(Q_GLOBAL, kv_sparse ? L_IDX : L_DENSE, p, s)) != BC_OK) return rc;
    ReduceParams r{};
    r.m = p.m; r.l = p.l; r.o = p.o; r.n_heads = H; r.n_splits = n_splits; r.head_dim = hd;
    r.out = a + size_t(b) * H * hd;
    if ((rc = launch_attn_reduce(r, s)) != BC_OK) return rc;
  }

  // S2 = top-k(a); o; h1 = bf16(h + o); x2 = RMSNorm(h1); S3; gate | up; f
  if ((rc = batch_proj(ly[0].w_o, H * hd, d, a, k_d, B, at_<int32_t>(ws, L.io), yo, gws, gws_bytes, s)) !=
      BC_OK)
    return rc;
  np = BatchNormParams{};
  np.h = hidden; np.add = yo; np.add_stride = d; np.h_out = hmid; np.gain = ly[0].g_mlp; np.d = d; np.eps = eps;
  np.x_out = x2;
  k_batch_norm<<<dim3(B), dim3(kBatchThreads), 0, s>>>(np);
  if ((rc = check_launch("k_batch_norm")) != BC_OK) return rc;
  if ((rc = batch_proj(ly[0].w_gu, d, 2 * dff, x2, k_d, B, at_<int32_t>(ws, L.igu), ygu, gws, gws_bytes,
                       s)) != BC_OK)
    return rc;
  k_batch_swiglu<<<dim3(unsigned(ceil_div(dff, 256)), B), dim3(256), 0, s>>>(ygu, dff, f);
  if ((rc = check_launch("k_batch_swiglu")) != BC_OK) return rc;
  // S4 = top-k(f); down; h = bf16(h1 + down)
  if ((rc = batch_proj(ly[0].w_down, dff, d, f, k_ff, B, at_<int32_t>(ws, L.idn), ydn, gws, gws_bytes,
                       s)) != BC_OK)
    return rc;
  k_batch_resid<<<dim3(unsigned(ceil_div(B * d, 256))), dim3(256), 0, s>>>(hmid, ydn, B * d, hidden);
  if ((rc = check_launch("k_batch_resid")) != BC_OK) return rc;

  if (taps) {
    const bool sp = k_d < d;
    // the channel lists are [batch][k] (one selection per sequence)
    for (int b = 0; b < B; ++b) {
      const bc_layer_taps& t = taps[b];
      if ((rc = copy_tap_b(t.x1, x1 + size_t(b) * d, size_t(d) * 2, s)) != BC_OK) return rc;
      if (sp && (rc = copy_tap_b(t.idx_qkv, at_<int32_t>(ws, L.i1) + size_t(b) * k_d, size_t(k_d) * 4, s)) != BC_OK)
        return rc;
      if ((rc = copy_tap_b(t.q, q + size_t(b) * H * hd, size_t(H) * hd * 2, s)) != BC_OK) return rc;
      for (int g = 0; g < Hkv && (t.k || t.v); ++g) {
        const size_t src = (size_t(g) * ly[b].n_cap + st->n_ctx - 1) * hd;
        if (t.k && (rc = copy_tap_b(t.k + size_t(g) * hd, ly[b].k_cache + src, size_t(hd) * 2, s)) != BC_OK) return rc;
        if (t.v && (rc = copy_tap_b(t.v + size_t(g) * hd, ly[b].v_cache + src, size_t(hd) * 2, s)) != BC_OK) return rc;
      }
      if (kv_sparse &&
          (rc = copy_tap_b(t.idx_kv, at_<int32_t>(ws, L.idx_kv) + size_t(b) * Hkv * n_sel, size_t(Hkv) * n_sel * 4,
                           s)) != BC_OK)
        return rc;
      if ((rc = copy_tap_b(t.a, a + size_t(b) * H * hd, size_t(H) * hd * 2, s)) != BC_OK) return rc;
      if (sp && (rc = copy_tap_b(t.idx_o, at_<int32_t>(ws, L.io) + size_t(b) * k_d, size_t(k_d) * 4, s)) != BC_OK)
        return rc;
      if ((rc = copy_tap_b(t.h_mid, hmid + size_t(b) * d, size_t(d) * 2, s)) != BC_OK) return rc;
      if ((rc = copy_tap_b(t.x2, x2 + size_t(b) * d, size_t(d) * 2, s)) != BC_OK) return rc;
      if (sp && (rc = copy_tap_b(t.idx_gu, at_<int32_t>(ws, L.igu) + size_t(b) * k_d, size_t(k_d) * 4, s)) != BC_OK)
        return rc;
      if ((rc = copy_tap_b(t.hff, f + size_t(b) * dff, size_t(dff) * 2, s)) != BC_OK) return rc;
      if (sp && (rc = copy_tap_b(t.idx_down, at_<int32_t>(ws, L.idn) + size_t(b) * k_ff, size_t(k_ff) * 4, s)) != BC_OK)
        return rc;
    }
  }
  return BC_OK;
}

int batch_splits(const bc_model_dims& m, const bc_step* st, const bc_kv_budget_info& bud) {
  const int n_sel = st->kv.r_kv < 1.0 ? bud.t_sel : st->n_ctx;
  return st->n_splits > 0 ? st->n_splits : bc_attn_default_splits(n_sel, m.n_kv_heads);
}

}  // namespace
}  // namespace bc

using namespace bc;

extern "C" size_t bc_layer_batch_workspace_bytes(const bc_model_dims* dims, int batch, int max_ctx, int max_splits) {
  if (!dims || batch < 1 || batch > kBatchSeqMax || max_ctx < 1 || max_splits < 1) return 0;
  if (dims->d <= 0 || dims->d_ff <= 0 || dims->n_heads <= 0 || dims->n_kv_heads <= 0 || dims->head_dim <= 0) return 0;
  return batch_layout(*dims, batch, max_ctx, max_splits).total;
}

extern "C" int bc_decode_layer_batch(const bc_model_dims* dims, const bc_layer* layers, int batch, const bc_step* st,
                                     uint16_t* hidden, const bc_layer_taps* taps, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!dims || !layers || !st || !hidden || !ws) return set_error(BC_ERR_INVALID, "bc_decode_layer_batch: NULL argument");
  int rc = check_batch_dims(dims);
  if (rc != BC_OK) return rc;
  if ((rc = check_batch_layers(*dims, layers, batch, st)) != BC_OK) return rc;
  bc_kv_budget_info bud;
  if ((rc = bc_kv_budget(st->n_ctx, &st->kv, &bud)) != BC_OK) return rc;
  const int S = batch_splits(*dims, st, bud);
  const BatchLayout L = batch_layout(*dims, batch, st->n_ctx, S);
  if (ws_bytes < L.total) return set_error(BC_ERR_WORKSPACE, "bc_decode_layer_batch: workspace %zu < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_error(BC_ERR_INVALID, "bc_decode_layer_batch: ws not 256-byte aligned");
  return batch_layer_body(*dims, layers, batch, st, bud, S, hidden, taps, ws, L, static_cast<hipStream_t>(stream));
}

extern "C" int bc_decode_step_batch(const bc_model_dims* dims, const bc_layer* layers, int n_layers, int batch,
                                    const uint16_t* g_final, const uint16_t* w_head, const bc_step* st,
                                    uint16_t* hidden, float* logits, int32_t* tokens, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!dims || !layers || n_layers < 1 || !g_final || !w_head || !st || !hidden || !logits || !tokens || !ws)
    return set_error(BC_ERR_INVALID, "bc_decode_step_batch: NULL argument or no layers");
  int rc = check_batch_dims(dims);
  if (rc != BC_OK) return rc;
  if (dims->vocab <= 0 || dims->vocab % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "bc_decode_step_batch: vocab %% 8 != 0");
  for (int i = 0; i < n_layers; ++i)
    if ((rc = check_batch_layers(*dims, layers + size_t(i) * batch, batch, st)) != BC_OK) return rc;
  bc_kv_budget_info bud;
  if ((rc = bc_kv_budget(st->n_ctx, &st->kv, &bud)) != BC_OK) return rc;
  const int S = batch_splits(*dims, st, bud);
  const BatchLayout L = batch_layout(*dims, batch, st->n_ctx, S);
  if (ws_bytes < L.total) return set_error(BC_ERR_WORKSPACE, "bc_decode_step_batch: workspace %zu < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_error(BC_ERR_INVALID, "bc_decode_step_batch: ws not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n_layers; ++i)
    if ((rc = batch_layer_body(*dims, layers + size_t(i) * batch, batch, st, bud, S, hidden, nullptr, ws, L, s)) != BC_OK)
      return rc;
  // final RMSNorm and the dense LM head, its weights read once for the batch
  BatchNormParams np{};
  np.h = hidden; np.gain = g_final; np.d = dims->d; np.eps = float(st->rms_eps); np.x_out = at_<uint16_t>(ws, L.x1);
  k_batch_norm<<<dim3(batch), dim3(kBatchThreads), 0, s>>>(np);
  if ((rc = check_launch("k_batch_norm")) != BC_OK) return rc;
  if ((rc = run_gemv_batch(w_head, 1, dims->d, dims->vocab, at_<uint16_t>(ws, L.x1), nullptr, dims->d, batch, nullptr,
                           logits, nullptr, at_<void>(ws, L.gws), L.total - L.gws, s)) != BC_OK)
    return rc;
  k_batch_argmax<<<dim3(batch), dim3(1024), 0, s>>>(logits, dims->vocab, tokens);
  return check_launch("k_batch_argmax");
}
