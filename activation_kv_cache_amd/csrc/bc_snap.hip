// bc_snap.hip -- the select-once KV policy in the SnapKV form, for gfx950.
//
// README FAQ "How is this different from TEAL and SnapKV?": the KV branch
// follows SnapKV and selects once, after prefill; README "Timing and quality
// on a GPU" and "API at a glance": the selection is then gathered into one
// buffer (select_and_compact; bc_kv_compact here) and read by the same dense
// split-K attention every step.
//
// For KV head g the R = w_obs * G observation rows (query i of the window at
// position n - w_obs + i, head j of the group) attend causally over the n
// cached tokens; a token's vote is its softmax weight summed over the rows.
// Votes are averaged over ks neighbouring tokens (zero outside [0, n)), and
// the k highest-scored history tokens of [sinks', n - window') are kept with
// the sinks and the window, ascending; equal scores keep the lower token.
//
// The logits Q_g K^T (R x n, inner dimension head_dim) are a dense
// contraction: each wave computes 32 rows x 32 tokens per tile with
// v_mfma_f32_32x32x16_bf16 (head_dim/16 steps), its query rows held in
// registers as the A operand and each lane loading 16 bytes of one key row
// per step as the B operand.  The softmax needs every row's max and sum over
// all tokens before any weight is known, so the keys are read twice:
//   k_snap_stats   per (token chunk, KV head): online max / sum per row
//                  (per lane, then merged over the 32 lanes of a row group)
//   k_snap_merge   per KV head: the chunks' (max, sum) merged per row
//   k_snap_votes   per (token chunk, KV head): weights exp(z - M) / L summed
//                  over the lane's rows, its partner half-wave and the waves
//   k_snap_select  per KV head (1024 lanes): pooled scores, an exact radix
//                  select of the k-th largest key (3 histogram passes over
//                  the candidates), then the kept tokens in index order.
// Accumulator layout of the 32x32 MFMA: lane l holds column l % 32 and, in
// register e (0..15), row 8 * (e / 4) + 4 * (l / 32) + e % 4.
#include <math.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSnapChunk = 512;       // tokens per work-group of the two key passes (16 tiles of 32)
constexpr int kSnapSelThreads = 1024;
constexpr int kSnapMaxRows = 256;     // w_obs * group

struct SnapParams {
  const uint16_t* q_obs;   // [w_obs][n_heads][D]
  const uint16_t* k_cache; // [n_kv_heads][n_cap][D]
  int n_cap, n_ctx, w_obs, n_heads, n_kv_heads, group, rows, n_chunks;
  float scale_log2;        // log2(e) / sqrt(D)
  float* stats;            // [n_kv_heads][n_chunks][rows][2]  (max, sum) in log2 units
  float* final_;           // [n_kv_heads][rows][2]            (max, 1 / sum)
  float* votes;            // [n_kv_heads][n_ctx]
  float* scores_out;       // optional [n_kv_heads][n_ctx] pooled
  int32_t* idx_out;        // [n_kv_heads][t_sel]
  int t_sel, k_tok, sinks, window, ks;
};

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// Row of accumulator register e for this lane (see the file header).
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// Query rows of wave w as MFMA A operands: row 32w + lane % 32, dims
// 16s + 8(lane / 32) .. +7 of step s.  Row r is query r / G of the window in
// head g*G + r % G.
template <int D>
__device__ __forceinline__ void load_rows(const SnapParams& p, int g, int w, int lane, bf16x8 (&a)[D / 16]) {
  const int r = 32 * w + (lane & 31);
  const int i = r / p.group, j = g * p.group + r % p.group;
  const uint16_t* q = p.q_obs + (size_t(i) * p.n_heads + j) * D + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) a[s] = load_bf16x8(q + 16 * s);
}

// Logits (unscaled) of the wave's 32 rows against tokens t0 .. t0+31; lane
// l's column is token t0 + l % 32 (zero keys past n).
template <int D>
__device__ __forceinline__ f32x16 tile_logits(const SnapParams& p, int g, int t0, int lane, const bf16x8 (&a)[D / 16]) {
  const int t = t0 + (lane & 31);
  const int tc = t < p.n_ctx ? t : p.n_ctx - 1;
  const uint16_t* k = p.k_cache + (size_t(g) * p.n_cap + tc) * D + 8 * (lane >> 5);
  bf16x8 b[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) b[s] = load_bf16x8(k + 16 * s);
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < D / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc, 0, 0, 0);
  return acc;
}

// (max, sum) pairs in log2 units merged: the larger max, sums rescaled to it.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  l = l * exp2f(m - M) + l2 * exp2f(m2 - M);
  m = M;
}

template <int D, int NW>
__global__ __launch_bounds__(NW * kWave) void k_snap_stats(const SnapParams p) {
  const int g = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bf16x8 a[D / 16];
  load_rows<D>(p, g, w, lane, a);
  int lim[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) lim[e] = p.n_ctx - p.w_obs + (32 * w + acc_row(e, lane)) / p.group;
  float m[16], l[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) { m[e] = -INFINITY; l[e] = 0.f; }
  const int c0 = chunk * kSnapChunk;
  const int c1 = min(c0 + kSnapChunk, p.n_ctx);
  for (int t0 = c0; t0 < c1; t0 += 32) {
    const f32x16 acc = tile_logits<D>(p, g, t0, lane, a);
    const int t = t0 + (lane & 31);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if (t < p.n_ctx && t <= lim[e]) {
        const float z = acc[e] * p.scale_log2;
        if (z > m[e]) { l[e] = l[e] * exp2f(m[e] - z) + 1.f; m[e] = z; }
        else l[e] += exp2f(z - m[e]);
      }
    }
  }
  // merge over the 32 lanes that hold the same rows (lane bits 0..4)
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float m2 = __shfl_xor(m[e], off, kWave), l2 = __shfl_xor(l[e], off, kWave);
      merge_ml(m[e], l[e], m2, l2);
    }
  }
  if ((lane & 31) == 0) {
    float* out = p.stats + ((size_t(g) * p.n_chunks + chunk) * p.rows + 32 * w) * 2;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      out[2 * acc_row(e, lane)] = m[e];
      out[2 * acc_row(e, lane) + 1] = l[e];
    }
  }
}

__global__ __launch_bounds__(kSnapMaxRows) void k_snap_merge(const SnapParams p) {
  const int g = blockIdx.x, r = threadIdx.x;
  if (r >= p.rows) return;
  float m = -INFINITY, l = 0.f;
  for (int c = 0; c < p.n_chunks; ++c) {
    const float* s = p.stats + ((size_t(g) * p.n_chunks + c) * p.rows + r) * 2;
    merge_ml(m, l, s[0], s[1]);
  }
  p.final_[(size_t(g) * p.rows + r) * 2] = m;
  p.final_[(size_t(g) * p.rows + r) * 2 + 1] = 1.f / l;   // l >= 1: token 0 is in every row's range
}

template <int D, int NW>
__global__ __launch_bounds__(NW * kWave) void k_snap_votes(const SnapParams p) {
  __shared__ float red[NW][32];
  const int g = blockIdx.y, chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bf16x8 a[D / 16];
  load_rows<D>(p, g, w, lane, a);
  int lim[16];
  float M[16], invL[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int r = 32 * w + acc_row(e, lane);
    lim[e] = p.n_ctx - p.w_obs + r / p.group;
    M[e] = p.final_[(size_t(g) * p.rows + r) * 2];
    invL[e] = p.final_[(size_t(g) * p.rows + r) * 2 + 1];
  }
  const int c0 = chunk * kSnapChunk;
  const int c1 = min(c0 + kSnapChunk, p.n_ctx);
  for (int t0 = c0; t0 < c1; t0 += 32) {
    const f32x16 acc = tile_logits<D>(p, g, t0, lane, a);
    const int t = t0 + (lane & 31);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      part += (t < p.n_ctx && t <= lim[e]) ? exp2f(acc[e] * p.scale_log2 - M[e]) * invL[e] : 0.f;
    part += __shfl_xor(part, 32, kWave);   // the other 16 rows of the wave's 32
    if (lane < 32) red[w][lane] = part;
    __syncthreads();
    if (w == 0 && lane < 32 && t < p.n_ctx) {
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) v += red[ww][lane];
      p.votes[size_t(g) * p.n_ctx + t] = v;
    }
    __syncthreads();
  }
}

// Pooled score of token t: the average of votes t - ks/2 .. t + ks/2 (zero
// outside [0, n)), summed in token order.
__device__ __forceinline__ float pooled(const float* v, int n, int t, int ks) {
  const int r = ks / 2;
  float acc = 0.f;
  for (int u = t - r; u <= t + r; ++u) acc += (u >= 0 && u < n) ? v[u] : 0.f;
  return acc / float(ks);
}

__global__ __launch_bounds__(kSnapSelThreads) void k_snap_select(const SnapParams p) {
  constexpr int NT = kSnapSelThreads, NW = NT / kWave, P = 8;
  __shared__ Topk32Smem<NT> sm;
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = p.n_ctx;
  const float* v = p.votes + size_t(g) * n;
  int32_t* out = p.idx_out + size_t(g) * p.t_sel;
  if (p.scores_out)
    for (int t = tid; t < n; t += NT) p.scores_out[size_t(g) * n + t] = pooled(v, n, t, p.ks);
  for (int t = tid; t < p.sinks; t += NT) out[t] = t;
  for (int t = tid; t < p.window; t += NT) out[p.sinks + p.k_tok + t] = n - p.window + t;
  const int lo = p.sinks, nc = n - p.window - p.sinks;
  if (p.k_tok <= 0) return;
  // exact k-th largest key: bits 31..21, then 20..8, then 7..0
  uint32_t prefix = 0, k_rem = uint32_t(p.k_tok);
  const int hi_bits[3] = {32, 21, 8};
  const int lo_bits[3] = {21, 8, 0};
  for (int pass = 0; pass < 3; ++pass) {
    {
      uint4* h4 = reinterpret_cast<uint4*>(sm.hist);
      for (int i = tid; i < 8192 / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    const int hb = hi_bits[pass], lb = lo_bits[pass];
    for (int c = tid; c < nc; c += NT) {
      const uint32_t key = float_order_key(pooled(v, n, lo + c, p.ks));
      const bool in = pass == 0 || (key >> (hb & 31)) == prefix;   // hb < 32 after the first pass
      if (in) atomicAdd(&sm.hist[(key >> lb) & ((1u << (hb - lb)) - 1u)], 1u);
    }
    __syncthreads();
    if (pass == 1) topk32_pick_bin<NT, 8192>(k_rem, sm);
    else topk32_pick_bin<NT, 2048>(k_rem, sm);
    prefix = (prefix << (hb - lb)) | sm.sel_bin;
    k_rem -= sm.sel_above;
    __syncthreads();
  }
  const uint32_t thr = prefix, need = k_rem;   // keep keys > thr and the first `need` equal to thr
  // the kept candidates in index order: chunks of NT * P, thread t holding
  // P consecutive ones; a block scan of (equal, greater) counts places them
  uint32_t tie_base = 0, out_base = 0;
  for (int cb = 0; cb < nc; cb += NT * P) {
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int c = cb + tid * P + e;
      if (c < nc) {
        const uint32_t key = float_order_key(pooled(v, n, lo + c, p.ks));
        gtm |= (key > thr ? 1u : 0u) << e;
        eqm |= (key == thr ? 1u : 0u) << e;
      }
    }
    const uint32_t gt = uint32_t(__popc(gtm)), eq = uint32_t(__popc(eqm));
    const uint32_t val = (eq << 16) | gt;
    const uint32_t inc = wave_scan_dpp(val);
    if (lane == kWave - 1) sm.whi[w] = inc;
    __syncthreads();
    uint32_t before, total;
    waves_before_total<NW>(sm.whi, __builtin_amdgcn_readfirstlane(w), &before, &total);
    before += inc - val;
    const uint32_t gt_b = before & 0xFFFFu, eq_b = before >> 16;
    uint32_t tb = tie_base + eq_b;   // equal keys before this thread
    uint32_t pos = out_base + gt_b + (min(tb, need) - min(tie_base, need));
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const bool is_gt = (gtm >> e) & 1u, is_eq = (eqm >> e) & 1u;
      if (is_gt || (is_eq && tb < need)) {
        if (pos < uint32_t(p.k_tok)) out[p.sinks + pos] = lo + cb + tid * P + e;   // always true: k_tok are kept
        ++pos;
      }
      if (is_eq) ++tb;
    }
    const uint32_t cgt = total & 0xFFFFu, ceq = total >> 16;
    out_base += cgt + (min(tie_base + ceq, need) - min(tie_base, need));
    tie_base += ceq;
    __syncthreads();   // whi is reused by the next chunk's scan
  }
}

template <int D, int NW>
int launch_passes(const SnapParams& p, hipStream_t s) {
  const dim3 grid(unsigned(p.n_chunks), unsigned(p.n_kv_heads));
  k_snap_stats<D, NW><<<grid, dim3(NW * kWave), 0, s>>>(p);
  int rc = check_launch("k_snap_stats");
  if (rc != BC_OK) return rc;
  k_snap_merge<<<dim3(unsigned(p.n_kv_heads)), dim3(kSnapMaxRows), 0, s>>>(p);
  if ((rc = check_launch("k_snap_merge")) != BC_OK) return rc;
  k_snap_votes<D, NW><<<grid, dim3(NW * kWave), 0, s>>>(p);
  return check_launch("k_snap_votes");
}

template <int D>
int launch_passes_d(int nw, const SnapParams& p, hipStream_t s) {
  switch (nw) {
    case 1: return launch_passes<D, 1>(p, s);
    case 2: return launch_passes<D, 2>(p, s);
    case 4: return launch_passes<D, 4>(p, s);
    case 8: return launch_passes<D, 8>(p, s);
    default: return set_error(BC_ERR_UNSUPPORTED, "snap: %d row waves", nw);
  }
}

struct SnapLayout { size_t stats, final_, votes, total; int n_chunks; };
SnapLayout snap_layout(int n_ctx, int n_kv_heads, int rows) {
  SnapLayout L;
  L.n_chunks = ceil_div(n_ctx, kSnapChunk);
  size_t off = 0;
  auto take = [&off](size_t bytes) { size_t o = off; off += align_up(bytes > 0 ? bytes : 1, 256); return o; };
  L.stats = take(size_t(n_kv_heads) * L.n_chunks * rows * 2 * 4);
  L.final_ = take(size_t(n_kv_heads) * rows * 2 * 4);
  L.votes = take(size_t(n_kv_heads) * n_ctx * 4);
  L.total = off;
  return L;
}

// Token budget of the select-once policy (tokens, not blocks).
void snap_budget(int n, const bc_kv_policy& pol, int* t_sel, int* k_tok, int* sp, int* wp) {
  long long T = static_cast<long long>(floor(pol.r_kv * double(n) + 0.5));
  if (T > n) T = n;
  if (T < 0) T = 0;
  const int t = int(T);
  *sp = pol.sinks < t ? pol.sinks : t;
  *wp = pol.window < t - *sp ? pol.window : t - *sp;
  *t_sel = t;
  *k_tok = t - *sp - *wp;
}

}  // namespace

}  // namespace bc

using namespace bc;

extern "C" int bc_kv_snap_t_sel(int n_ctx, const bc_kv_policy* pol) {
  if (!pol || n_ctx < 0 || pol->sinks < 0 || pol->window < 0 || !(pol->r_kv >= 0.0))
    return set_error(BC_ERR_INVALID, "bc_kv_snap_t_sel: bad arguments");
  if (pol->r_kv >= 1.0) return n_ctx;
  int t_sel, k, sp, wp;
  snap_budget(n_ctx, *pol, &t_sel, &k, &sp, &wp);
  return t_sel;
}

extern "C" size_t bc_kv_snap_select_workspace_bytes(int n_ctx, int n_heads, int n_kv_heads, int w_obs) {
  if (n_ctx < 1 || n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0 || w_obs < 1) return 0;
  const int rows = w_obs * (n_heads / n_kv_heads);
  if (rows % 32 != 0 || rows > kSnapMaxRows) return 0;
  return snap_layout(n_ctx, n_kv_heads, rows).total;
}

extern "C" int bc_kv_snap_select(const uint16_t* q_obs, int w_obs, const uint16_t* k_cache, int n_cap, int n_ctx,
                                 int n_heads, int n_kv_heads, int head_dim, const bc_kv_policy* pol, int pool_kernel,
                                 int32_t* idx_out, float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q_obs || !k_cache || !pol || !idx_out || !ws) return set_error(BC_ERR_INVALID, "bc_kv_snap_select: NULL pointer");
  if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return set_error(BC_ERR_INVALID, "bc_kv_snap_select: heads %d / %d", n_heads, n_kv_heads);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "bc_kv_snap_select: head_dim %d", head_dim);
  if (n_ctx < 1 || n_ctx > n_cap) return set_error(BC_ERR_INVALID, "bc_kv_snap_select: n_ctx=%d n_cap=%d", n_ctx, n_cap);
  if (w_obs < 1 || w_obs > n_ctx) return set_error(BC_ERR_INVALID, "bc_kv_snap_select: w_obs=%d", w_obs);
  const int G = n_heads / n_kv_heads, rows = w_obs * G;
  if (rows % 32 != 0 || rows > kSnapMaxRows)
    return set_error(BC_ERR_UNSUPPORTED, "bc_kv_snap_select: w_obs * group = %d must be a multiple of 32 up to %d",
                     rows, kSnapMaxRows);
  if (pool_kernel < 1 || pool_kernel > 63 || pool_kernel % 2 == 0)
    return set_error(BC_ERR_INVALID, "bc_kv_snap_select: pool_kernel=%d (odd, 1..63)", pool_kernel);
  if (pol->sinks < 0 || pol->window < 0 || !(pol->r_kv >= 0.0))
    return set_error(BC_ERR_INVALID, "bc_kv_snap_select: sinks/window/r_kv out of range");
  if (pol->r_kv >= 1.0) return set_error(BC_ERR_INVALID, "bc_kv_snap_select: r_kv >= 1 needs no selection");
  const SnapLayout L = snap_layout(n_ctx, n_kv_heads, rows);
  if (ws_bytes < L.total) return set_error(BC_ERR_WORKSPACE, "bc_kv_snap_select: workspace %zu < %zu", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return set_error(BC_ERR_INVALID, "bc_kv_snap_select: ws not 256-byte aligned");
  if ((reinterpret_cast<uintptr_t>(q_obs) | reinterpret_cast<uintptr_t>(k_cache)) & 15)
    return set_error(BC_ERR_INVALID, "bc_kv_snap_select: q_obs and k_cache must be 16-byte aligned");
  SnapParams p{};
  p.q_obs = q_obs; p.k_cache = k_cache; p.n_cap = n_cap; p.n_ctx = n_ctx; p.w_obs = w_obs;
  p.n_heads = n_heads; p.n_kv_heads = n_kv_heads; p.group = G; p.rows = rows; p.n_chunks = L.n_chunks;
  p.scale_log2 = float(1.4426950408889634 / sqrt(double(head_dim)));
  char* base = static_cast<char*>(ws);
  p.stats = reinterpret_cast<float*>(base + L.stats);
  p.final_ = reinterpret_cast<float*>(base + L.final_);
  p.votes = reinterpret_cast<float*>(base + L.votes);
  p.scores_out = scores_out;
  p.idx_out = idx_out;
  p.ks = pool_kernel;
  snap_budget(n_ctx, *pol, &p.t_sel, &p.k_tok, &p.sinks, &p.window);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nw = rows / 32;
  int rc = head_dim == 128 ? launch_passes_d<128>(nw, p, s) : launch_passes_d<64>(nw, p, s);
  if (rc != BC_OK) return rc;
  k_snap_select<<<dim3(unsigned(n_kv_heads)), dim3(kSnapSelThreads), 0, s>>>(p);
  return check_launch("k_snap_select");
}
