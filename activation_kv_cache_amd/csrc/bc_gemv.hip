// bc_gemv.hip -- activation-sparse projection GEMV for gfx950.
//
// y[o] = sum_{j<k} W^T[idx_j][o] * x[idx_j]  (README "What it does in one
// picture": each token's activations select the weight columns read).
//
// W^T is [d_in][d_out] bf16: the weights of one input channel are one
// contiguous row.  The main kernel gives a work-group a 128-column tile of y
// (256 B of every row) and a fixed chunk of the selected channel list.  Its
// 256 lanes form 16 row slots of 16 lanes; a slot reads one row's 256 B per
// load (16 B per lane), 8 rows in flight per slot, so a work-group keeps
// 128 rows (32 KB) in flight.  The chunk's channel ids and their x values are
// staged in LDS first.  Each work-group writes its fp32 partial sums for its
// chunk; no work-group waits for another (cross-XCD fences on this chip cost
// far more than a kernel boundary).  A finish kernel then adds the chunks in
// chunk order -- deterministic -- and applies the epilogue: bf16 store,
// residual add + RMSNorm + top-k of the next input (one work-group), rotary +
// KV append + block summary, or SwiGLU (+ top-k).  With a single chunk the
// main kernel stores bf16 or fp32 (+ per-tile argmax) directly.
// Dense mode is the same kernel with idx == NULL.
#include <math.h>
#include <stdlib.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

constexpr int kSlots = kGemvThreads / 16;   // 16 row slots of 16 lanes
constexpr int kRowsInFlight = 8;            // per slot
constexpr int kStageRows = 1024;            // channel ids / x values staged per pass

struct MainSmem {
  int32_t ch[kStageRows];
  float xv[kStageRows];
  float red[kSlots][kGemvTile];
  float amax_v[kGemvThreads / kWave];
  int32_t amax_i[kGemvThreads / kWave];
};

template <int MODE>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_main(const GemvParams p) {
  __shared__ MainSmem sm;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x;
  const int l16 = tid & 15, slot = tid >> 4;
  const int col = tile * kGemvTile + l16 * 8;
  const bool col_ok = col < p.d_out;
  const int r0 = split * p.rows_per_split;
  const int r1 = min(p.k, r0 + p.rows_per_split);

  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  // plain: row ch of W^T at wt + ch * d_out; tile-major: the tile's rows are
  // contiguous, each as wide as the tile
  const int tile_w = min(kGemvTile, p.d_out - tile * kGemvTile);
  const uint16_t* wcol;
  size_t row_stride;
  if (p.tiled) {
    wcol = p.wt + size_t(tile) * kGemvTile * p.d_in + (col_ok ? l16 * 8 : 0);
    row_stride = size_t(tile_w);
  } else {
    wcol = p.wt + (col_ok ? col : 0);
    row_stride = size_t(p.d_out);
  }
  const bool dense = p.idx == nullptr;

  for (int s0 = r0; s0 < r1; s0 += kStageRows) {
    const int s1 = min(r1, s0 + kStageRows);
    const int n = s1 - s0;
    // dense rows are known before staging: put the first batch in flight now
    uint4 wv[kRowsInFlight];
    if (dense) {
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int rr = slot + kSlots * u;
        wv[u] = (col_ok && rr < n) ? *reinterpret_cast<const uint4*>(wcol + size_t(s0 + rr) * row_stride)
                                   : make_uint4(0, 0, 0, 0);
      }
    }
    for (int r = s0 + tid; r < s1; r += kGemvThreads) {
      const int ch = dense ? r : p.idx[r];
      sm.ch[r - s0] = ch;
      sm.xv[r - s0] = bf16_to_f32(p.x[ch]);
    }
    __syncthreads();
    for (int r = slot; r < n; r += kSlots * kRowsInFlight) {
      float xv[kRowsInFlight];
      if (!dense || r != slot) {
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) {
          const int rr = r + kSlots * u;
          wv[u] = (col_ok && rr < n) ? *reinterpret_cast<const uint4*>(wcol + size_t(sm.ch[rr]) * row_stride)
                                     : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        const int rr = r + kSlots * u;
        xv[u] = rr < n ? sm.xv[rr] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kRowsInFlight; ++u) {
        acc[0] += bf16_lo(wv[u].x) * xv[u];
        acc[1] += bf16_hi(wv[u].x) * xv[u];
        acc[2] += bf16_lo(wv[u].y) * xv[u];
        acc[3] += bf16_hi(wv[u].y) * xv[u];
        acc[4] += bf16_lo(wv[u].z) * xv[u];
        acc[5] += bf16_hi(wv[u].z) * xv[u];
        acc[6] += bf16_lo(wv[u].w) * xv[u];
        acc[7] += bf16_hi(wv[u].w) * xv[u];
      }
    }
    __syncthreads();
  }

  // slots 0..15 in order
  float4* rw = reinterpret_cast<float4*>(&sm.red[slot][l16 * 8]);
  rw[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  rw[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  float v = 0.f;
  int c = -1;
  if (tid < kGemvTile) {
#pragma unroll
    for (int s = 0; s < kSlots; ++s) v += sm.red[s][tid];
    c = tile * kGemvTile + tid;
    if (c >= p.d_out) c = -1;
  }
  if constexpr (MODE == MAIN_PARTIAL) {
    if (c >= 0) p.partial[size_t(split) * p.d_out + c] = v;
  } else if constexpr (MODE == MAIN_BF16) {
    if (c >= 0) p.y[c] = f32_to_bf16(v);
  } else if constexpr (MODE == MAIN_F32_ARGMAX) {
    float best = -INFINITY;
    int besti = 0x7FFFFFFF;
    if (c >= 0) {
      p.yf[c] = v;
      best = v;
      besti = c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(best, off, kWave);
      const int oi = __shfl_xor(besti, off, kWave);
      if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
    }
    if ((tid & 63) == 0) { sm.amax_v[tid >> 6] = best; sm.amax_i[tid >> 6] = besti; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kGemvThreads / kWave; ++w) {
        const float ov = sm.amax_v[w];
        const int oi = sm.amax_i[w];
        if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
      }
      p.tile_max[tile] = best;
      p.tile_arg[tile] = besti;
    }
  }
}

// ------------------------------------------------------------------ finish
// Sum of the n_splits chunk partials of column c, in chunk order.
__device__ __forceinline__ float chunk_sum(const float* partial, int n_splits, int d_out, int c) {
  float v = 0.f;
  int s = 0;
  for (; s + 4 <= n_splits; s += 4) {
    const float a0 = partial[size_t(s) * d_out + c];
    const float a1 = partial[size_t(s + 1) * d_out + c];
    const float a2 = partial[size_t(s + 2) * d_out + c];
    const float a3 = partial[size_t(s + 3) * d_out + c];
    v += a0; v += a1; v += a2; v += a3;
  }
  for (; s < n_splits; ++s) v += partial[size_t(s) * d_out + c];
  return v;
}

// Same for 4 consecutive columns (c % 4 == 0, d_out % 8 == 0).
__device__ __forceinline__ float4 chunk_sum4(const float* partial, int n_splits, int d_out, int c) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* pp = partial + c;
  int s = 0;
  for (; s + 4 <= n_splits; s += 4) {
    const float4 a0 = *reinterpret_cast<const float4*>(pp + size_t(s) * d_out);
    const float4 a1 = *reinterpret_cast<const float4*>(pp + size_t(s + 1) * d_out);
    const float4 a2 = *reinterpret_cast<const float4*>(pp + size_t(s + 2) * d_out);
    const float4 a3 = *reinterpret_cast<const float4*>(pp + size_t(s + 3) * d_out);
    v.x += a0.x; v.y += a0.y; v.z += a0.z; v.w += a0.w;
    v.x += a1.x; v.y += a1.y; v.z += a1.z; v.w += a1.w;
    v.x += a2.x; v.y += a2.y; v.z += a2.z; v.w += a2.w;
    v.x += a3.x; v.y += a3.y; v.z += a3.z; v.w += a3.w;
  }
  for (; s < n_splits; ++s) {
    const float4 a0 = *reinterpret_cast<const float4*>(pp + size_t(s) * d_out);
    v.x += a0.x; v.y += a0.y; v.z += a0.z; v.w += a0.w;
  }
  return v;
}

__global__ __launch_bounds__(256) void k_finish_bf16(const FinishParams p) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < p.d_out) p.y[c] = f32_to_bf16(chunk_sum(p.partial, p.n_splits, p.d_out, c));
}

// Rotary (rotate-half) cos/sin of pair i at position pos.  The angle
// pos * theta^(-2i/D) is formed in double and reduced by 2*pi in double
// (two-part constant), so single-precision sincos of the reduced angle is
// accurate to float rounding at any position.
__device__ __forceinline__ void rope_cs(int pos, double log2_theta, int i, int D, float* cs, float* sn) {
  const double inv_freq = exp2(-2.0 * double(i) / double(D) * log2_theta);
  const double ang = double(pos) * inv_freq;
  const double kq = rint(ang * 0.15915494309189533577);
  double r = fma(-kq, 6.28318530717958623200, ang);
  r = fma(-kq, 2.44929359829470635445e-16, r);
  sincosf(float(r), sn, cs);
}

// One work-group per head of the q | k | v output: thread i owns the pair
// (i, i + D/2).  q -> q_out; k, v -> cache slot pos; then the (min, max)
// summary of block pos/16 is recomputed for the key heads.
__global__ __launch_bounds__(64) void k_finish_qkv(const FinishParams p) {
  const int D = p.head_dim, half = D / 2;
  const int head = blockIdx.x;
  const int qh = p.n_heads, kvh = p.n_kv_heads;
  const int base = head * D;
  for (int i = threadIdx.x; i < half; i += 64) {
    float a = chunk_sum(p.partial, p.n_splits, p.d_out, base + i);
    float b = chunk_sum(p.partial, p.n_splits, p.d_out, base + i + half);
    if (head < qh + kvh) {
      float cs, sn;
      rope_cs(p.pos, p.log2_theta, i, D, &cs, &sn);
      const float ra = a * cs - b * sn;
      const float rb = b * cs + a * sn;
      a = ra;
      b = rb;
    }
    const uint16_t ba = f32_to_bf16(a), bb = f32_to_bf16(b);
    if (head < qh) {
      p.q_out[base + i] = ba;
      p.q_out[base + i + half] = bb;
    } else if (head < qh + kvh) {
      const int g = head - qh;
      uint16_t* kr = p.k_cache + (size_t(g) * p.n_cap + p.pos) * D;
      kr[i] = ba;
      kr[i + half] = bb;
      if (p.summary != nullptr) {
        const int blk = p.pos / 16;
        const uint16_t* kc = p.k_cache + size_t(g) * p.n_cap * D;
        uint16_t* sp = p.summary + (size_t(g) * (p.n_cap / 16) + blk) * D * 2;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int dd = e ? i + half : i;
          const uint16_t nb = e ? bb : ba;
          uint16_t rows[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) rows[t] = blk * 16 + t < p.pos ? kc[size_t(blk * 16 + t) * D + dd] : nb;
          uint16_t bmn = nb, bmx = nb;
          float mn = bf16_to_f32(nb), mx = mn;
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const float f = bf16_to_f32(rows[t]);
            if (f < mn) { mn = f; bmn = rows[t]; }
            if (f > mx) { mx = f; bmx = rows[t]; }
          }
          sp[dd * 2 + 0] = bmn;
          sp[dd * 2 + 1] = bmx;
        }
      }
    } else {
      const int g = head - qh - kvh;
      uint16_t* vr = p.v_cache + (size_t(g) * p.n_cap + p.pos) * D;
      vr[i] = ba;
      vr[i + half] = bb;
    }
  }
}

constexpr int kOneGroup = 1024;

struct OneGroupSmem {
  union {
    TopkSmem<kOneGroup, uint16_t> topk;
    Topk15Smem topk15;
  };
  float part[kOneGroup / kWave];
};

// Sum of squares of bf16 x[0..n) with a fixed order (thread-strided partial
// sums, wave butterfly, waves in order).  All threads get the total.
__device__ float one_group_sum_squares(const uint16_t* x, int n, float* part) {
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += kOneGroup) {
    const float v = bf16_to_f32(x[i]);
    s += v * v;
  }
  s = wave_sum_f32(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kOneGroup / kWave; ++w) t += part[w];
  __syncthreads();
  return t;
}

__device__ void one_group_select(const uint16_t* x, int n, int k, int32_t* idx_out, OneGroupSmem& sm) {
  auto key = [x](int i) -> uint32_t { return uint32_t(x[i]) & 0x7FFFu; };
  auto emit = [idx_out](int r, int i) { idx_out[r] = i; };
  if (n <= kTopk15MaxN)
    block_topk15(n, k, key, emit, sm.topk15);
  else
    block_topk<kOneGroup, 15, uint16_t>(n, k, key, emit, sm.topk);
}

// One work-group: y = bf16(resid + sum of chunks); then optionally
// x_next = RMSNorm(y) * gain and the top-k of x_next.
__global__ __launch_bounds__(kOneGroup) void k_finish_resid(const FinishParams p) {
  __shared__ OneGroupSmem sm;
  for (int c = threadIdx.x * 4; c < p.d_out; c += kOneGroup * 4) {
    const float4 v = chunk_sum4(p.partial, p.n_splits, p.d_out, c);
    float r[4] = {v.x, v.y, v.z, v.w};
    if (p.resid) {
      const uint2 rr = *reinterpret_cast<const uint2*>(p.resid + c);
      r[0] += bf16_lo(rr.x); r[1] += bf16_hi(rr.x); r[2] += bf16_lo(rr.y); r[3] += bf16_hi(rr.y);
    }
    uint2 o;
    o.x = uint32_t(f32_to_bf16(r[0])) | (uint32_t(f32_to_bf16(r[1])) << 16);
    o.y = uint32_t(f32_to_bf16(r[2])) | (uint32_t(f32_to_bf16(r[3])) << 16);
    *reinterpret_cast<uint2*>(p.y + c) = o;
  }
  __syncthreads();
  if (p.norm_gain == nullptr) return;
  const float ss = one_group_sum_squares(p.y, p.d_out, sm.part);
  const float inv = 1.0f / sqrtf(ss / float(p.d_out) + p.eps);
  for (int c = threadIdx.x; c < p.d_out; c += kOneGroup)
    p.x_next[c] = f32_to_bf16(bf16_to_f32(p.y[c]) * inv * bf16_to_f32(p.norm_gain[c]));
  __syncthreads();
  if (p.sel_k > 0 && p.sel_k < p.d_out) one_group_select(p.x_next, p.d_out, p.sel_k, p.idx_next, sm);
}

// SwiGLU over the packed gate | up chunks: tile t holds gate columns
// [128t, 128t + w) and up columns [128t + w, 128t + 2w) of hidden units
// [64t, 64t + w), w = min(64, d_ff - 64t).  One work-group when a top-k of
// the result follows, else one thread per hidden unit.
__global__ __launch_bounds__(kOneGroup) void k_finish_swiglu(const FinishParams p) {
  __shared__ OneGroupSmem sm;
  const int half = kGemvTile / 2;
  const int stride = gridDim.x * kOneGroup * 4;
  for (int u = (blockIdx.x * kOneGroup + threadIdx.x) * 4; u < p.d_ff; u += stride) {
    const int t = u / half, off = u % half;
    const int w = min(half, p.d_ff - t * half);
    const float4 gt = chunk_sum4(p.partial, p.n_splits, p.d_out, t * kGemvTile + off);
    const float4 up = chunk_sum4(p.partial, p.n_splits, p.d_out, t * kGemvTile + w + off);
    const float g[4] = {gt.x, gt.y, gt.z, gt.w};
    const float v[4] = {up.x, up.y, up.z, up.w};
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(g[e] / (1.0f + expf(-g[e])) * v[e]);
    uint2 ov;
    ov.x = uint32_t(o[0]) | (uint32_t(o[1]) << 16);
    ov.y = uint32_t(o[2]) | (uint32_t(o[3]) << 16);
    *reinterpret_cast<uint2*>(p.y + u) = ov;
  }
  if (p.sel_k <= 0 || p.sel_k >= p.d_ff) return;
  __syncthreads();
  one_group_select(p.y, p.d_ff, p.sel_k, p.idx_next, sm);
}

__global__ __launch_bounds__(256) void k_argmax_finish(const float* tile_max, const int32_t* tile_arg, int n_tiles,
                                                      int32_t* token) {
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  float best = -INFINITY;
  int besti = 0x7FFFFFFF;
  for (int t = threadIdx.x; t < n_tiles; t += 256) {
    const float v = tile_max[t];
    const int i = tile_arg[t];
    if (v > best || (v == best && i < besti)) { best = v; besti = i; }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best, off, kWave);
    const int oi = __shfl_xor(besti, off, kWave);
    if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = besti; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sv[w] > best || (sv[w] == best && si[w] < besti)) { best = sv[w]; besti = si[w]; }
    *token = besti;
  }
}

__global__ __launch_bounds__(kOneGroup) void k_select(const uint16_t* x, int n, int k, int32_t* idx_out) {
  __shared__ OneGroupSmem sm;
  one_group_select(x, n, k, idx_out, sm);
}

__global__ __launch_bounds__(kOneGroup) void k_norm_select(const uint16_t* h, const uint16_t* g, int d, float eps,
                                                          uint16_t* x_out, int k, int32_t* idx_out) {
  __shared__ OneGroupSmem sm;
  const float ss = one_group_sum_squares(h, d, sm.part);
  const float inv = 1.0f / sqrtf(ss / float(d) + eps);
  for (int i = threadIdx.x; i < d; i += kOneGroup)
    x_out[i] = f32_to_bf16(bf16_to_f32(h[i]) * inv * bf16_to_f32(g[i]));
  __syncthreads();
  if (idx_out != nullptr && k > 0 && k < d) one_group_select(x_out, d, k, idx_out, sm);
}

}  // namespace

static int gemv_target_groups() {
  // tuning override for sweeps; the default is the measured best
  static const int v = [] {
    const char* e = getenv("BC_GEMV_GROUPS");
    const int x = e ? atoi(e) : 0;
    return x > 0 ? x : 512;
  }();
  return v;
}

GemvPlan plan_gemv(int d_out, int k) {
  GemvPlan pl;
  pl.n_tiles = ceil_div(d_out, kGemvTile);
  const int target_groups = gemv_target_groups();
  int splits = ceil_div(target_groups, pl.n_tiles);
  const int max_splits = k > 0 ? ceil_div(k, 64) : 1;   // at least 64 rows per chunk
  if (splits > max_splits) splits = max_splits;
  if (splits > 32) splits = 32;
  if (splits < 1) splits = 1;
  int rps = ceil_div(k > 0 ? k : 1, splits);
  rps = (rps + 15) / 16 * 16;
  pl.rows_per_split = rps;
  pl.n_splits = k > 0 ? ceil_div(k, rps) : 1;
  pl.partial_bytes = align_up(size_t(pl.n_splits) * d_out * 4, 256);
  return pl;
}

int launch_gemv_main(int mode, const GemvParams& p, hipStream_t s) {
  dim3 grid(p.n_tiles, p.n_splits), block(kGemvThreads);
  switch (mode) {
    case MAIN_PARTIAL: k_gemv_main<MAIN_PARTIAL><<<grid, block, 0, s>>>(p); break;
    case MAIN_BF16: k_gemv_main<MAIN_BF16><<<grid, block, 0, s>>>(p); break;
    case MAIN_F32_ARGMAX: k_gemv_main<MAIN_F32_ARGMAX><<<grid, block, 0, s>>>(p); break;
    default: return set_error(BC_ERR_INVALID, "unknown GEMV mode %d", mode);
  }
  return check_launch("k_gemv_main");
}

int launch_finish(int kind, const FinishParams& p, hipStream_t s) {
  switch (kind) {
    case FIN_BF16: k_finish_bf16<<<ceil_div(p.d_out, 256), 256, 0, s>>>(p); break;
    case FIN_QKV: k_finish_qkv<<<p.n_heads + 2 * p.n_kv_heads, 64, 0, s>>>(p); break;
    case FIN_RESID: k_finish_resid<<<1, kOneGroup, 0, s>>>(p); break;
    case FIN_SWIGLU: {
      const bool sel = p.sel_k > 0 && p.sel_k < p.d_ff;
      k_finish_swiglu<<<sel ? 1 : ceil_div(p.d_ff, kOneGroup * 4), kOneGroup, 0, s>>>(p);
      break;
    }
    default: return set_error(BC_ERR_INVALID, "unknown finish kind %d", kind);
  }
  return check_launch("k_finish");
}

int launch_argmax_finish(const float* tile_max, const int32_t* tile_arg, int n_tiles, int32_t* token, hipStream_t s) {
  k_argmax_finish<<<1, 256, 0, s>>>(tile_max, tile_arg, n_tiles, token);
  return check_launch("k_argmax_finish");
}

int launch_norm_select(const uint16_t* h, const uint16_t* g, int d, float eps, uint16_t* x_out, int k,
                       int32_t* idx_out, hipStream_t s) {
  k_norm_select<<<1, kOneGroup, 0, s>>>(h, g, d, eps, x_out, k, idx_out);
  return check_launch("k_norm_select");
}

int launch_select(const uint16_t* x, int n, int k, int32_t* idx_out, hipStream_t s) {
  k_select<<<1, kOneGroup, 0, s>>>(x, n, k, idx_out);
  return check_launch("k_select");
}

}  // namespace bc

using namespace bc;

extern "C" size_t bc_sparse_gemv_workspace_bytes(int d_out, int k) {
  if (d_out <= 0 || k <= 0) return 0;
  GemvPlan pl = plan_gemv(d_out, k);
  return pl.n_splits > 1 ? pl.partial_bytes : 256;
}

static int sparse_gemv_impl(const uint16_t* wt, int tiled, int d_in, int d_out, const uint16_t* x,
                            const int32_t* idx, int k, uint16_t* y, void* ws, size_t ws_bytes, void* stream,
                            const char* name) {
  if (!wt || !x || !y) return set_error(BC_ERR_INVALID, "%s: NULL pointer", name);
  if (d_in <= 0 || d_out <= 0) return set_error(BC_ERR_INVALID, "%s: d_in=%d d_out=%d", name, d_in, d_out);
  if (d_out % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "%s: d_out %% 8 != 0 (%d)", name, d_out);
  if (idx == nullptr) {
    if (k != d_in) return set_error(BC_ERR_INVALID, "%s: dense call needs k == d_in", name);
  } else if (k < 1 || k > d_in) {
    return set_error(BC_ERR_INVALID, "%s: k=%d outside [1, %d]", name, k, d_in);
  }
  if ((reinterpret_cast<uintptr_t>(wt) | reinterpret_cast<uintptr_t>(ws)) & 15)
    return set_error(BC_ERR_INVALID, "%s: wt and ws must be 16-byte aligned", name);
  GemvPlan pl = plan_gemv(d_out, k);
  const size_t need = bc_sparse_gemv_workspace_bytes(d_out, k);
  if (!ws || ws_bytes < need) return set_error(BC_ERR_WORKSPACE, "%s: workspace %zu < %zu", name, ws_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemvParams p{};
  p.wt = wt; p.tiled = tiled; p.d_in = d_in; p.d_out = d_out; p.x = x; p.idx = idx; p.k = k;
  p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
  p.partial = static_cast<float*>(ws);
  p.y = y;
  if (pl.n_splits == 1) return launch_gemv_main(MAIN_BF16, p, s);
  int rc = launch_gemv_main(MAIN_PARTIAL, p, s);
  if (rc != BC_OK) return rc;
  FinishParams f{};
  f.partial = p.partial; f.n_splits = pl.n_splits; f.d_out = d_out; f.y = y;
  return launch_finish(FIN_BF16, f, s);
}

extern "C" int bc_sparse_gemv(const uint16_t* wt, int d_in, int d_out, const uint16_t* x, const int32_t* idx,
                              int k, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  return sparse_gemv_impl(wt, 0, d_in, d_out, x, idx, k, y, ws, ws_bytes, stream, "bc_sparse_gemv");
}

extern "C" int bc_sparse_gemv_tiled(const uint16_t* wt_packed, int d_in, int d_out, const uint16_t* x,
                                    const int32_t* idx, int k, uint16_t* y, void* ws, size_t ws_bytes,
                                    void* stream) {
  return sparse_gemv_impl(wt_packed, 1, d_in, d_out, x, idx, k, y, ws, ws_bytes, stream, "bc_sparse_gemv_tiled");
}
