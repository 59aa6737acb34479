// bc_masked.hip -- the masked-attention dense baseline, for gfx950.
//
// README FAQ "A KV method reports a speedup above its byte bound": measured
// against a dense step whose attention is masked rather than split-K, a KV
// policy looks several times faster than it is (the abstract: near five).
// This is that baseline: decode attention computed the way a plain
// masked attention does it over a preallocated cache -- scores of every query
// head against every slot of the cache, a mask of -inf on the slots past the
// context, a softmax over the whole row, then the weighted sum of every value
// row -- with the scores and the weights materialised in HBM between the
// steps, and each query head reading the keys and values of its KV head
// itself (no sharing across the query heads of a group).
//
//   k_mask_scores   z[j][t] = scale * q_j . k_t for every slot t < n_cap
//                   (-inf for t >= n_ctx); one work-group per (256 slots,
//                   query head), 16 bytes of a key row per lane
//   k_mask_softmax  p[j][t] = e^(z - max) / sum e^(z - max), in place; one
//                   work-group per query head, three passes over the row
//   k_mask_pv       partial[j][s] = sum over the split's slots of p * v_t
//   k_mask_sum      out[j] = bf16(sum over splits, in split order)
// Every kernel reads and writes with coalesced 16-byte accesses; the waste is
// in the algorithm (whole-capacity rows, per-head re-reads, round trips of
// the score matrix), which is what the baseline is for.
#include <math.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2m(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

constexpr int kMaskThreads = 256;
constexpr int kMaskTile = 256;          // slots per work-group of the score pass
constexpr int kMaskSoftThreads = 1024;
constexpr int kMaskPvSlots = 1024;      // slots per split of the value pass (at least)
constexpr int kMaskMaxSplits = 64;

struct MaskParams {
  const uint16_t* q;       // [H][D]
  const uint16_t* k_cache; // [Hkv][n_cap][D]
  const uint16_t* v_cache;
  int n_cap, n_ctx, n_heads, n_kv_heads, head_dim, n_splits, split_len;
  float scale;
  float* scores;           // [H][n_cap]: z, then p
  float* partial;          // [H][n_splits][D]
  uint16_t* out;           // [H][D]
};

// Sum over the LPT lanes of a row group (LPT in {8, 16}), every lane of the
// group ending with it.
template <int LPT>
__device__ __forceinline__ float row_group_sum(float v) {
  return group_sum<LPT>(v);
}

template <int D>
__global__ __launch_bounds__(kMaskThreads) void k_mask_scores(const MaskParams p) {
  constexpr int LPT = D / 8;                     // lanes per key row, 16 bytes each
  constexpr int RPI = kMaskThreads / LPT;        // rows per work-group iteration
  const int j = blockIdx.y, g = j / (p.n_heads / p.n_kv_heads);
  const int r = threadIdx.x % LPT, sub = threadIdx.x / LPT;
  const uint4 qv = *reinterpret_cast<const uint4*>(p.q + size_t(j) * D + 8 * r);
  const uint16_t* Kg = p.k_cache + size_t(g) * p.n_cap * D + 8 * r;
  float* zrow = p.scores + size_t(j) * p.n_cap;
  const int t0 = blockIdx.x * kMaskTile;
#pragma unroll
  for (int i = 0; i < kMaskTile / RPI; ++i) {
    const int t = t0 + i * RPI + sub;
    const int tc = t < p.n_cap ? t : p.n_cap - 1;
    const uint4 kv = *reinterpret_cast<const uint4*>(Kg + size_t(tc) * D);
    float acc = dot2m(qv.x, kv.x, 0.f);
    acc = dot2m(qv.y, kv.y, acc);
    acc = dot2m(qv.z, kv.z, acc);
    acc = dot2m(qv.w, kv.w, acc);
    acc = row_group_sum<LPT>(acc);
    if (r == 0 && t < p.n_cap) zrow[t] = t < p.n_ctx ? acc * p.scale : -INFINITY;
  }
}

// Block reductions over 16 waves through LDS, in wave order.
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < kMaskSoftThreads / kWave; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  return m;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum_f32(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < kMaskSoftThreads / kWave; ++i) s += red[i];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(kMaskSoftThreads) void k_mask_softmax(const MaskParams p) {
  __shared__ float red[kMaskSoftThreads / kWave];
  float4* row = reinterpret_cast<float4*>(p.scores + size_t(blockIdx.x) * p.n_cap);
  const int n4 = p.n_cap / 4;
  float m = -INFINITY;
  for (int i = threadIdx.x; i < n4; i += kMaskSoftThreads) {
    const float4 z = row[i];
    m = fmaxf(m, fmaxf(fmaxf(z.x, z.y), fmaxf(z.z, z.w)));
  }
  const float M = block_max(m, red);
  float s = 0.f;
  for (int i = threadIdx.x; i < n4; i += kMaskSoftThreads) {
    const float4 z = row[i];
    s += (expf(z.x - M) + expf(z.y - M)) + (expf(z.z - M) + expf(z.w - M));
  }
  const float inv = 1.0f / block_sum(s, red);
  for (int i = threadIdx.x; i < n4; i += kMaskSoftThreads) {
    const float4 z = row[i];
    row[i] = make_float4(expf(z.x - M) * inv, expf(z.y - M) * inv, expf(z.z - M) * inv, expf(z.w - M) * inv);
  }
}

template <int D>
__global__ __launch_bounds__(kMaskThreads) void k_mask_pv(const MaskParams p) {
  constexpr int LPT = D / 8;
  constexpr int RPI = kMaskThreads / LPT;
  __shared__ float red[RPI][D + 4];
  const int j = blockIdx.y, s = blockIdx.x, g = j / (p.n_heads / p.n_kv_heads);
  const int r = threadIdx.x % LPT, sub = threadIdx.x / LPT;
  const uint16_t* Vg = p.v_cache + size_t(g) * p.n_cap * D + 8 * r;
  const float* prow = p.scores + size_t(j) * p.n_cap;
  const int c0 = s * p.split_len, c1 = min(p.n_cap, c0 + p.split_len);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int t = c0 + sub; t < c1; t += RPI) {
    const float w = prow[t];
    const uint4 v = *reinterpret_cast<const uint4*>(Vg + size_t(t) * D);
    acc[0] = fmaf(w, bf16_lo(v.x), acc[0]);
    acc[1] = fmaf(w, bf16_hi(v.x), acc[1]);
    acc[2] = fmaf(w, bf16_lo(v.y), acc[2]);
    acc[3] = fmaf(w, bf16_hi(v.y), acc[3]);
    acc[4] = fmaf(w, bf16_lo(v.z), acc[4]);
    acc[5] = fmaf(w, bf16_hi(v.z), acc[5]);
    acc[6] = fmaf(w, bf16_lo(v.w), acc[6]);
    acc[7] = fmaf(w, bf16_hi(v.w), acc[7]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[sub][8 * r + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float v = 0.f;
    for (int i = 0; i < RPI; ++i) v += red[i][threadIdx.x];
    p.partial[(size_t(j) * p.n_splits + s) * D + threadIdx.x] = v;
  }
}

__global__ __launch_bounds__(128) void k_mask_sum(const MaskParams p) {
  const int j = blockIdx.x, d = threadIdx.x;
  if (d >= p.head_dim) return;
  float v = 0.f;
  for (int s = 0; s < p.n_splits; ++s) v += p.partial[(size_t(j) * p.n_splits + s) * p.head_dim + d];
  p.out[size_t(j) * p.head_dim + d] = f32_to_bf16(v);
}

int mask_splits(int n_cap) { return max(1, min(kMaskMaxSplits, n_cap / kMaskPvSlots)); }

struct MaskLayout { size_t scores, partial, total; };
MaskLayout mask_layout(int n_cap, int n_heads, int head_dim) {
  MaskLayout L;
  L.scores = 0;
  L.partial = align_up(size_t(n_heads) * n_cap * 4, 256);
  L.total = L.partial + align_up(size_t(n_heads) * mask_splits(n_cap) * head_dim * 4, 256);
  return L;
}

}  // namespace

size_t masked_attn_workspace(int n_cap, int n_heads, int head_dim) {
  return mask_layout(n_cap, n_heads, head_dim).total;
}

int launch_masked_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int n_cap, int n_ctx,
                       int n_heads, int n_kv_heads, int head_dim, float scale, uint16_t* out, void* ws,
                       hipStream_t s) {
  const MaskLayout L = mask_layout(n_cap, n_heads, head_dim);
  MaskParams p{};
  p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.n_cap = n_cap; p.n_ctx = n_ctx;
  p.n_heads = n_heads; p.n_kv_heads = n_kv_heads; p.head_dim = head_dim; p.scale = scale;
  p.n_splits = mask_splits(n_cap);
  p.split_len = ceil_div(n_cap, p.n_splits);
  p.scores = reinterpret_cast<float*>(static_cast<char*>(ws) + L.scores);
  p.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + L.partial);
  p.out = out;
  const dim3 sgrid(unsigned(ceil_div(n_cap, kMaskTile)), unsigned(n_heads));
  const dim3 pgrid(unsigned(p.n_splits), unsigned(n_heads));
  if (head_dim == 128) {
    k_mask_scores<128><<<sgrid, dim3(kMaskThreads), 0, s>>>(p);
  } else {
    k_mask_scores<64><<<sgrid, dim3(kMaskThreads), 0, s>>>(p);
  }
  int rc = check_launch("k_mask_scores");
  if (rc != BC_OK) return rc;
  k_mask_softmax<<<dim3(unsigned(n_heads)), dim3(kMaskSoftThreads), 0, s>>>(p);
  if ((rc = check_launch("k_mask_softmax")) != BC_OK) return rc;
  if (head_dim == 128) {
    k_mask_pv<128><<<pgrid, dim3(kMaskThreads), 0, s>>>(p);
  } else {
    k_mask_pv<64><<<pgrid, dim3(kMaskThreads), 0, s>>>(p);
  }
  if ((rc = check_launch("k_mask_pv")) != BC_OK) return rc;
  k_mask_sum<<<dim3(unsigned(n_heads)), dim3(128), 0, s>>>(p);
  return check_launch("k_mask_sum");
}

}  // namespace bc

using namespace bc;

extern "C" size_t bc_masked_attn_workspace_bytes(int n_cap, int n_heads, int head_dim) {
  if (n_cap < 16 || n_cap % 16 != 0 || n_heads <= 0 || !valid_head_dim(head_dim)) return 0;
  return masked_attn_workspace(n_cap, n_heads, head_dim);
}

extern "C" int bc_masked_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, int n_cap,
                              int n_ctx, int n_heads, int n_kv_heads, int head_dim, float scale, uint16_t* out,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !out || !ws) return set_error(BC_ERR_INVALID, "bc_masked_attn: NULL pointer");
  if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return set_error(BC_ERR_INVALID, "bc_masked_attn: heads %d / %d", n_heads, n_kv_heads);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "bc_masked_attn: head_dim %d", head_dim);
  if (n_cap < 16 || n_cap % 16 != 0 || n_ctx < 1 || n_ctx > n_cap)
    return set_error(BC_ERR_INVALID, "bc_masked_attn: n_cap=%d n_ctx=%d", n_cap, n_ctx);
  const size_t need = masked_attn_workspace(n_cap, n_heads, head_dim);
  if (ws_bytes < need) return set_error(BC_ERR_WORKSPACE, "bc_masked_attn: workspace %zu < %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) ||
      ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) &
       15))
    return set_error(BC_ERR_INVALID, "bc_masked_attn: misaligned pointer");
  return launch_masked_attn(q, k_cache, v_cache, n_cap, n_ctx, n_heads, n_kv_heads, head_dim, scale, out, ws,
                            static_cast<hipStream_t>(stream));
}
