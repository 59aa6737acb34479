// bc_gemv.hip -- activation-sparse projection GEMV for gfx950.
//
// y[o] = sum_{j<k} W^T[idx_j][o] * x[idx_j]  (README "What it does in one
// picture": each token's activations select the weight columns read).
//
// Layout: W^T is [d_in][d_out] bf16, so the weights of one selected input
// channel are one contiguous row.  A work-group owns a 512-column tile of y
// and a fixed chunk of the selected channel list: each of its 4 waves walks
// every 4th selected row, one 16-byte load per lane (a wave reads 1 KB of a
// row per instruction), 8 rows in flight per wave.  Partial sums of the
// chunks go to an fp32 workspace; the last work-group of a tile (atomic
// counter) adds them in chunk order -- deterministic -- and applies the
// epilogue (bf16 store, residual add, rotary + KV append, SwiGLU, fp32 +
// argmax).  Optionally the last tile to finish runs a tail on the whole
// output (top-k selection for the next GEMV, RMSNorm + selection, argmax).
// Dense mode is the same kernel with idx == NULL.
#include <math.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

constexpr int kRowsInFlight = 8;

struct GemvSmem {
  union {
    float red[4][kGemvTile];          // per-wave sums
    float half[2][kGemvTile];         // split-sum halves
    TopkSmem<kGemvThreads> topk;      // tail selection
    struct { float v[kGemvThreads / kWave]; int32_t i[kGemvThreads / kWave]; } amax;
    float norm_part[kGemvThreads / kWave];
  } u;
  float tile[kGemvTile];
  int flag;
};

// Sum of squares of x[0..n) in fp32 with a fixed order: thread-strided
// partial sums, then a wave tree, then waves in order.
__device__ float block_sum_squares(const uint16_t* x, int n, float* wave_part) {
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += kGemvThreads) {
    float v = bf16_to_f32(x[i]);
    s += v * v;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
  if (wave_lane() == 0) wave_part[threadIdx.x >> 6] = s;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kGemvThreads / kWave; ++w) t += wave_part[w];
  __syncthreads();
  return t;
}

__device__ void tail_select(const uint16_t* x, int n, int k, int32_t* idx_out, GemvSmem& sm) {
  auto key = [x](int i) -> uint32_t { return uint32_t(x[i]) & 0x7FFFu; };
  auto emit = [idx_out](int r, int i) { idx_out[r] = i; };
  block_topk<kGemvThreads, 15>(n, k, key, emit, sm.u.topk);
}

template <int EPI>
__device__ void epilogue(const GemvParams& p, int tile, GemvSmem& sm) {
  const int tid = threadIdx.x;
  const int base = tile * kGemvTile;
  if constexpr (EPI == EPI_BF16 || EPI == EPI_RESID) {
    for (int c = tid; c < kGemvTile; c += kGemvThreads) {
      int col = base + c;
      if (col >= p.d_out) break;
      float v = sm.tile[c];
      if constexpr (EPI == EPI_RESID) v += bf16_to_f32(p.resid[col]);
      p.y[col] = f32_to_bf16(v);
    }
  } else if constexpr (EPI == EPI_F32_ARGMAX) {
    float best = -INFINITY;
    int besti = 0x7FFFFFFF;
    for (int c = tid; c < kGemvTile; c += kGemvThreads) {
      int col = base + c;
      if (col >= p.d_out) break;
      float v = sm.tile[c];
      p.yf[col] = v;
      if (v > best || (v == best && col < besti)) { best = v; besti = col; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(best, off, kWave);
      int oi = __shfl_xor(besti, off, kWave);
      if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
    }
    if (wave_lane() == 0) { sm.u.amax.v[tid >> 6] = best; sm.u.amax.i[tid >> 6] = besti; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < kGemvThreads / kWave; ++w) {
        float ov = sm.u.amax.v[w];
        int oi = sm.u.amax.i[w];
        if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
      }
      p.tile_max[tile] = best;
      p.tile_arg[tile] = besti;
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int D = p.head_dim, half = D / 2;
    const int qdim = p.n_heads * D, kvdim = p.n_kv_heads * D;
    for (int c = tid; c < kGemvTile; c += kGemvThreads) {
      int col = base + c;
      if (col >= p.d_out) break;
      float v = sm.tile[c];
      if (col < qdim + kvdim) {
        // rotary, rotate-half pairs (i, i + D/2) of the column's head
        int i = col % D;
        int ip = i < half ? i : i - half;
        double ang = double(p.pos) * pow(p.theta, -2.0 * double(ip) / double(D));
        float cs = float(cos(ang)), sn = float(sin(ang));
        float other = sm.tile[i < half ? c + half : c - half];
        v = i < half ? v * cs - other * sn : v * cs + other * sn;
      }
      uint16_t b = f32_to_bf16(v);
      if (col < qdim) {
        p.q_out[col] = b;
      } else if (col < qdim + kvdim) {
        int g = (col - qdim) / D, i = (col - qdim) % D;
        p.k_cache[(size_t(g) * p.n_cap + p.pos) * D + i] = b;
      } else {
        int g = (col - qdim - kvdim) / D, i = (col - qdim - kvdim) % D;
        p.v_cache[(size_t(g) * p.n_cap + p.pos) * D + i] = b;
      }
    }
    if (p.summary != nullptr) {
      __syncthreads();
      // refresh (min, max) of block pos/16 for the key heads in this tile
      const int blk = p.pos / 16;
      for (int c = tid; c < kGemvTile; c += kGemvThreads) {
        int col = base + c;
        if (col >= p.d_out || col < qdim || col >= qdim + kvdim) continue;
        int g = (col - qdim) / D, i = (col - qdim) % D;
        // the new key, rounded as stored
        int ip = i < half ? i : i - half;
        double ang = double(p.pos) * pow(p.theta, -2.0 * double(ip) / double(D));
        float cs = float(cos(ang)), sn = float(sin(ang));
        float other = sm.tile[i < half ? c + half : c - half];
        float kv = i < half ? sm.tile[c] * cs - other * sn : sm.tile[c] * cs + other * sn;
        uint16_t kb = f32_to_bf16(kv);
        float mn = bf16_to_f32(kb), mx = mn;
        uint16_t bmn = kb, bmx = kb;
        const uint16_t* kc = p.k_cache + size_t(g) * p.n_cap * D + i;
        for (int t = blk * 16; t < p.pos; ++t) {
          uint16_t u = kc[size_t(t) * D];
          float f = bf16_to_f32(u);
          if (f < mn) { mn = f; bmn = u; }
          if (f > mx) { mx = f; bmx = u; }
        }
        uint16_t* sp = p.summary + ((size_t(g) * (p.n_cap / 16) + blk) * D + i) * 2;
        sp[0] = bmn;
        sp[1] = bmx;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // tile t holds gate columns [0, w) then up columns [w, 2w) of group t
    const int w = min(kGemvTile / 2, p.d_ff - tile * (kGemvTile / 2));
    for (int c = tid; c < w; c += kGemvThreads) {
      float gt = sm.tile[c], up = sm.tile[w + c];
      float silu = gt / (1.0f + expf(-gt));
      p.y[tile * (kGemvTile / 2) + c] = f32_to_bf16(silu * up);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(const GemvParams p) {
  __shared__ GemvSmem sm;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = wave_lane(), w = wave_id();
  const int col = tile * kGemvTile + lane * 8;
  const bool col_ok = col < p.d_out;
  const int r0 = split * p.rows_per_split;
  const int r1 = min(p.k, r0 + p.rows_per_split);

  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;

  const uint16_t* wcol = p.wt + col;
  for (int r = r0 + w; r < r1; r += 4 * kRowsInFlight) {
    uint4 wv[kRowsInFlight];
    float xv[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int rr = r + 4 * u;
      if (rr < r1) {
        const int ch = p.idx ? __builtin_amdgcn_readfirstlane(p.idx[rr]) : rr;
        xv[u] = bf16_to_f32(p.x[ch]);
        wv[u] = col_ok ? *reinterpret_cast<const uint4*>(wcol + size_t(ch) * p.d_out) : make_uint4(0, 0, 0, 0);
      } else {
        xv[u] = 0.f;
        wv[u] = make_uint4(0, 0, 0, 0);
      }
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

  // waves 0..3 in order
  float4* rw = reinterpret_cast<float4*>(&sm.u.red[w][lane * 8]);
  rw[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  rw[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  float v0, v1;
  {
    const int c = tid * 2;
    v0 = ((sm.u.red[0][c] + sm.u.red[1][c]) + sm.u.red[2][c]) + sm.u.red[3][c];
    v1 = ((sm.u.red[0][c + 1] + sm.u.red[1][c + 1]) + sm.u.red[2][c + 1]) + sm.u.red[3][c + 1];
  }
  if (p.n_splits == 1) {
    sm.tile[tid * 2] = v0;
    sm.tile[tid * 2 + 1] = v1;
  } else {
    const int c = tile * kGemvTile + tid * 2;
    if (c < p.d_out)
      *reinterpret_cast<float2*>(p.partial + size_t(split) * p.d_out + c) = make_float2(v0, v1);
    __threadfence();
    __syncthreads();
    if (tid == 0) sm.flag = atomicAdd(&p.counters[tile], 1u) == unsigned(p.n_splits - 1);
    __syncthreads();
    if (!sm.flag) return;
    __threadfence();
    // add the chunks in chunk order: two halves, each sequential, then half0 + half1
    const int cg = tid & 127, hf = tid >> 7;
    const int smid = (p.n_splits + 1) / 2;
    const int s0 = hf ? smid : 0, s1 = hf ? p.n_splits : smid;
    const int cc = tile * kGemvTile + cg * 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cc < p.d_out) {
      const float* pp = p.partial + cc;
      int s = s0;
      for (; s + 4 <= s1; s += 4) {
        float4 b0 = *reinterpret_cast<const float4*>(pp + size_t(s) * p.d_out);
        float4 b1 = *reinterpret_cast<const float4*>(pp + size_t(s + 1) * p.d_out);
        float4 b2 = *reinterpret_cast<const float4*>(pp + size_t(s + 2) * p.d_out);
        float4 b3 = *reinterpret_cast<const float4*>(pp + size_t(s + 3) * p.d_out);
        a.x += b0.x; a.y += b0.y; a.z += b0.z; a.w += b0.w;
        a.x += b1.x; a.y += b1.y; a.z += b1.z; a.w += b1.w;
        a.x += b2.x; a.y += b2.y; a.z += b2.z; a.w += b2.w;
        a.x += b3.x; a.y += b3.y; a.z += b3.z; a.w += b3.w;
      }
      for (; s < s1; ++s) {
        float4 b0 = *reinterpret_cast<const float4*>(pp + size_t(s) * p.d_out);
        a.x += b0.x; a.y += b0.y; a.z += b0.z; a.w += b0.w;
      }
    }
    __syncthreads();   // red[] is no longer read; half[] aliases it
    *reinterpret_cast<float4*>(&sm.u.half[hf][cg * 4]) = a;
    __syncthreads();
    for (int c = tid; c < kGemvTile; c += kGemvThreads) sm.tile[c] = sm.u.half[0][c] + sm.u.half[1][c];
    if (tid == 0) p.counters[tile] = 0u;
  }
  __syncthreads();
  epilogue<EPI>(p, tile, sm);

  if (p.tail == TAIL_NONE) return;
  __threadfence();
  __syncthreads();
  if (tid == 0) sm.flag = atomicAdd(&p.counters[p.n_tiles], 1u) == unsigned(p.n_tiles - 1);
  __syncthreads();
  if (!sm.flag) return;
  __threadfence();
  if (tid == 0) p.counters[p.n_tiles] = 0u;

  if (p.tail == TAIL_SELECT) {
    tail_select(p.tail_in, p.tail_n, p.tail_k, p.tail_idx_out, sm);
  } else if (p.tail == TAIL_NORM_SELECT) {
    float ss = block_sum_squares(p.tail_in, p.tail_n, sm.u.norm_part);
    const float inv = 1.0f / sqrtf(ss / float(p.tail_n) + p.tail_eps);
    for (int i = tid; i < p.tail_n; i += kGemvThreads)
      p.tail_x_out[i] = f32_to_bf16(bf16_to_f32(p.tail_in[i]) * inv * bf16_to_f32(p.tail_gain[i]));
    __syncthreads();
    if (p.tail_k < p.tail_n) tail_select(p.tail_x_out, p.tail_n, p.tail_k, p.tail_idx_out, sm);
  } else if (p.tail == TAIL_ARGMAX) {
    float best = -INFINITY;
    int besti = 0x7FFFFFFF;
    for (int t = tid; t < p.n_tiles; t += kGemvThreads) {
      float v = p.tile_max[t];
      int i = p.tile_arg[t];
      if (v > best || (v == best && i < besti)) { best = v; besti = i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(best, off, kWave);
      int oi = __shfl_xor(besti, off, kWave);
      if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
    }
    if (wave_lane() == 0) { sm.u.amax.v[tid >> 6] = best; sm.u.amax.i[tid >> 6] = besti; }
    __syncthreads();
    if (tid == 0) {
      for (int w2 = 1; w2 < kGemvThreads / kWave; ++w2) {
        float ov = sm.u.amax.v[w2];
        int oi = sm.u.amax.i[w2];
        if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
      }
      *p.token_out = besti;
    }
  }
}

}  // namespace

GemvPlan plan_gemv(int d_out, int k) {
  GemvPlan pl;
  pl.n_tiles = ceil_div(d_out, kGemvTile);
  const int target_groups = 1024;     // about 4 work-groups per compute unit
  int splits = ceil_div(target_groups, pl.n_tiles);
  const int max_splits = k > 0 ? ceil_div(k, 32) : 1;   // at least 32 rows per chunk
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int rps = ceil_div(k > 0 ? k : 1, splits);
  rps = (rps + 3) / 4 * 4;
  pl.rows_per_split = rps;
  pl.n_splits = k > 0 ? ceil_div(k, rps) : 1;
  pl.counter_bytes = align_up(size_t(pl.n_tiles + 1) * 4, 256);
  pl.partial_bytes = pl.n_splits > 1 ? align_up(size_t(pl.n_splits) * d_out * 4, 256) : 0;
  return pl;
}

int launch_gemv(int epi, const GemvParams& p, hipStream_t s) {
  dim3 grid(p.n_tiles, p.n_splits), block(kGemvThreads);
  switch (epi) {
    case EPI_BF16: k_gemv<EPI_BF16><<<grid, block, 0, s>>>(p); break;
    case EPI_F32_ARGMAX: k_gemv<EPI_F32_ARGMAX><<<grid, block, 0, s>>>(p); break;
    case EPI_RESID: k_gemv<EPI_RESID><<<grid, block, 0, s>>>(p); break;
    case EPI_QKV: k_gemv<EPI_QKV><<<grid, block, 0, s>>>(p); break;
    case EPI_SWIGLU: k_gemv<EPI_SWIGLU><<<grid, block, 0, s>>>(p); break;
    default: return set_error(BC_ERR_INVALID, "unknown GEMV epilogue %d", epi);
  }
  return check_launch("k_gemv");
}

}  // namespace bc

using namespace bc;

extern "C" size_t bc_sparse_gemv_workspace_bytes(int d_out, int k) {
  if (d_out <= 0 || k <= 0) return 0;
  GemvPlan pl = plan_gemv(d_out, k);
  return pl.counter_bytes + pl.partial_bytes;
}

extern "C" int bc_sparse_gemv(const uint16_t* wt, int d_in, int d_out, const uint16_t* x, const int32_t* idx,
                              int k, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!wt || !x || !y) return set_error(BC_ERR_INVALID, "bc_sparse_gemv: NULL pointer");
  if (d_in <= 0 || d_out <= 0) return set_error(BC_ERR_INVALID, "bc_sparse_gemv: d_in=%d d_out=%d", d_in, d_out);
  if (d_out % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "bc_sparse_gemv: d_out %% 8 != 0 (%d)", d_out);
  if (idx == nullptr) {
    if (k != d_in) return set_error(BC_ERR_INVALID, "bc_sparse_gemv: dense call needs k == d_in");
  } else if (k < 1 || k > d_in) {
    return set_error(BC_ERR_INVALID, "bc_sparse_gemv: k=%d outside [1, %d]", k, d_in);
  }
  if ((reinterpret_cast<uintptr_t>(wt) | reinterpret_cast<uintptr_t>(ws)) & 15)
    return set_error(BC_ERR_INVALID, "bc_sparse_gemv: wt and ws must be 16-byte aligned");
  GemvPlan pl = plan_gemv(d_out, k);
  if (!ws || ws_bytes < pl.counter_bytes + pl.partial_bytes)
    return set_error(BC_ERR_WORKSPACE, "bc_sparse_gemv: workspace %zu < %zu", ws_bytes,
                     pl.counter_bytes + pl.partial_bytes);
  GemvParams p{};
  p.wt = wt; p.d_in = d_in; p.d_out = d_out; p.x = x; p.idx = idx; p.k = k;
  p.rows_per_split = pl.rows_per_split; p.n_splits = pl.n_splits; p.n_tiles = pl.n_tiles;
  p.counters = static_cast<uint32_t*>(ws);
  p.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.counter_bytes);
  p.y = y;
  p.tail = TAIL_NONE;
  return launch_gemv(EPI_BF16, p, static_cast<hipStream_t>(stream));
}
