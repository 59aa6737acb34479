// bc_attn.hip -- split-K grouped-query decode attention for gfx950.
//
// README "Overview": dense and sparse modes read their caches through the
// same split-K attention kernel, so the dense baseline stays fixed.  Here the
// dense mode is the same kernel with idx == NULL.
//
// Partial pass: one work-group per (split, KV head).  A key (value) row is
// head_dim bf16 = 256 B at head_dim 128; 16 lanes hold one row (16 B each),
// so one wave load covers 4 consecutive list positions (1 KB contiguous in
// dense mode and inside a selected 16-token block).  The G query heads of the
// KV head live in registers as bf16 pairs; q.k uses v_dot2 (bf16 pairs into
// fp32) and a DPP sum over the 16 lanes.  Each group of 16 lanes keeps its
// own online-softmax state (m, l, o) in log2 units; the 16 states of a
// work-group are merged through LDS at the end.  In index mode the split's
// slice of the index list is staged in LDS.
//
// Merge pass: M = max m_s, out = sum o_s e^(m_s-M) / sum l_s e^(m_s-M),
// one work-group per query head.
#include <math.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

constexpr int kAttnThreads = 256;
constexpr int kIdxChunk = 1024;
constexpr float kLn2 = 0.693147180559945309f;

template <int D, int G>
struct AttnSmem {
  static constexpr int LPT = D / 8;
  static constexpr int SLOTS = (kAttnThreads / kWave) * (kWave / LPT);
  float o[SLOTS][G][D];
  float m[SLOTS][G];
  float l[SLOTS][G];
  int32_t idx[kIdxChunk];
};

template <int D, int G>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(const AttnParams p) {
  constexpr int LPT = D / 8;          // lanes per row
  constexpr int TPL = kWave / LPT;    // rows per wave load
  constexpr int U = 16 / TPL;         // loads per iteration: 16 positions per wave iteration
  constexpr int TPI = TPL * U;
  __shared__ AttnSmem<D, G> sm;

  const int s = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = wave_lane(), w = wave_id();
  const int sub = lane / LPT, r = lane % LPT;
  const int c = (p.n_sel + p.n_splits - 1) / p.n_splits;
  const int lo = s * c;
  const int hi = min(p.n_sel, lo + c);

  uint32_t qv[G][4];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    uint4 t = *reinterpret_cast<const uint4*>(p.q + size_t(g * G + j) * D + r * 8);
    qv[j][0] = t.x; qv[j][1] = t.y; qv[j][2] = t.z; qv[j][3] = t.w;
  }
  float m_run[G], l_run[G], o_acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o_acc[j][e] = 0.f;
  }

  const uint16_t* Kg = p.k_cache + size_t(g) * p.n_cap * D + r * 8;
  const uint16_t* Vg = p.v_cache + size_t(g) * p.n_cap * D + r * 8;
  const int32_t* idxg = p.idx ? p.idx + size_t(g) * p.n_sel : nullptr;

  for (int c0 = lo; c0 < hi; c0 += kIdxChunk) {
    const int c1 = min(hi, c0 + kIdxChunk);
    if (idxg) {
      for (int i = tid; i < c1 - c0; i += kAttnThreads) sm.idx[i] = idxg[c0 + i];
      __syncthreads();
    }
    for (int base = c0 + w * TPI; base < c1; base += (kAttnThreads / kWave) * TPI) {
      uint4 kr[U], vr[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int pos = base + u * TPL + sub;
        valid[u] = pos < c1;
        int pc = valid[u] ? pos : c1 - 1;
        int t = idxg ? sm.idx[pc - c0] : pc;
        kr[u] = *reinterpret_cast<const uint4*>(Kg + size_t(t) * D);
        vr[u] = *reinterpret_cast<const uint4*>(Vg + size_t(t) * D);
      }
      float z[G][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float a = dot2(qv[j][0], kr[u].x, 0.f);
          a = dot2(qv[j][1], kr[u].y, a);
          a = dot2(qv[j][2], kr[u].z, a);
          a = dot2(qv[j][3], kr[u].w, a);
          a = group_sum<LPT>(a);
          z[j][u] = valid[u] ? a * p.scale_log2 : -INFINITY;
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float mt = z[j][0];
#pragma unroll
        for (int u = 1; u < U; ++u) mt = fmaxf(mt, z[j][u]);
        const float mn = fmaxf(m_run[j], mt);
        const float alpha = m_run[j] == -INFINITY ? 0.f : exp2f(m_run[j] - mn);
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o_acc[j][e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float pu = valid[u] ? exp2f(z[j][u] - mn) : 0.f;
          psum += pu;
          o_acc[j][0] += pu * bf16_lo(vr[u].x);
          o_acc[j][1] += pu * bf16_hi(vr[u].x);
          o_acc[j][2] += pu * bf16_lo(vr[u].y);
          o_acc[j][3] += pu * bf16_hi(vr[u].y);
          o_acc[j][4] += pu * bf16_lo(vr[u].z);
          o_acc[j][5] += pu * bf16_hi(vr[u].z);
          o_acc[j][6] += pu * bf16_lo(vr[u].w);
          o_acc[j][7] += pu * bf16_hi(vr[u].w);
        }
        l_run[j] = l_run[j] * alpha + psum;
        m_run[j] = mn;
      }
    }
    if (idxg) __syncthreads();
  }

  // merge the work-group's lane-group states
  const int slot = w * TPL + sub;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float4* dst = reinterpret_cast<float4*>(&sm.o[slot][j][r * 8]);
    dst[0] = make_float4(o_acc[j][0], o_acc[j][1], o_acc[j][2], o_acc[j][3]);
    dst[1] = make_float4(o_acc[j][4], o_acc[j][5], o_acc[j][6], o_acc[j][7]);
    if (r == 0) { sm.m[slot][j] = m_run[j]; sm.l[slot][j] = l_run[j]; }
  }
  __syncthreads();
  constexpr int SLOTS = AttnSmem<D, G>::SLOTS;
  for (int e = tid; e < G * D; e += kAttnThreads) {
    const int j = e / D, d = e % D;
    float M = -INFINITY;
    for (int q = 0; q < SLOTS; ++q) M = fmaxf(M, sm.m[q][j]);
    float acc = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
      for (int q = 0; q < SLOTS; ++q) {
        const float mq = sm.m[q][j];
        if (mq == -INFINITY) continue;
        const float wq = exp2f(mq - M);
        acc += sm.o[q][j][d] * wq;
        lsum += sm.l[q][j] * wq;
      }
    }
    const int jh = g * G + j;
    p.o[(size_t(jh) * p.n_splits + s) * D + d] = acc;
    if (d == 0) {
      p.m[size_t(jh) * p.n_splits + s] = M == -INFINITY ? -INFINITY : M * kLn2;
      p.l[size_t(jh) * p.n_splits + s] = lsum;
    }
  }
}

// One work-group per query head.  M and the weights w_s = e^(m_s - M) are
// computed once into LDS; the weighted sums over splits are split between
// thread groups (fixed halves) and combined in a fixed order.
constexpr int kReduceMaxSplits = 4096;

__global__ __launch_bounds__(kAttnThreads) void k_attn_reduce(const ReduceParams p) {
  __shared__ float wts[kReduceMaxSplits];
  __shared__ float part[kAttnThreads];
  __shared__ float red[kAttnThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = blockIdx.x;
  const int D = p.head_dim, S = p.n_splits;
  const float* mj = p.m + size_t(j) * S;
  const float* lj = p.l + size_t(j) * S;
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kAttnThreads) mx = fmaxf(mx, mj[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  if (lane == 0) red[w] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < kAttnThreads / kWave; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float den = 0.f;
  for (int s = tid; s < S; s += kAttnThreads) {
    const float ms = mj[s];
    const float wt = (ms == -INFINITY || M == -INFINITY) ? 0.f : expf(ms - M);
    wts[s] = wt;
    den += wt * lj[s];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off, kWave);
  if (lane == 0) red[w] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int i = 0; i < kAttnThreads / kWave; ++i) den += red[i];
  const int groups = kAttnThreads / D;          // 2 at head_dim 128, 4 at 64
  const int grp = tid / D, d = tid % D;
  const int per = (S + groups - 1) / groups;
  const int s0 = min(S, grp * per), s1 = min(S, s0 + per);
  const float* oj = p.o + size_t(j) * S * D + d;
  float num = 0.f;
  int s = s0;
  for (; s + 4 <= s1; s += 4) {
    const float o0 = oj[size_t(s) * D], o1 = oj[size_t(s + 1) * D];
    const float o2 = oj[size_t(s + 2) * D], o3 = oj[size_t(s + 3) * D];
    num += o0 * wts[s];
    num += o1 * wts[s + 1];
    num += o2 * wts[s + 2];
    num += o3 * wts[s + 3];
  }
  for (; s < s1; ++s) num += oj[size_t(s) * D] * wts[s];
  part[tid] = num;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int g = 0; g < groups; ++g) t += part[g * D + tid];
    p.out[size_t(j) * D + tid] = f32_to_bf16(den > 0.f ? t / den : 0.f);
  }
}

template <int D>
int launch_partial_d(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.n_splits, p.n_kv_heads), block(kAttnThreads);
  switch (p.n_heads / p.n_kv_heads) {
    case 1: k_attn_partial<D, 1><<<grid, block, 0, s>>>(p); break;
    case 2: k_attn_partial<D, 2><<<grid, block, 0, s>>>(p); break;
    case 4: k_attn_partial<D, 4><<<grid, block, 0, s>>>(p); break;
    case 8: k_attn_partial<D, 8><<<grid, block, 0, s>>>(p); break;
    default: return set_error(BC_ERR_UNSUPPORTED, "attention: group size %d", p.n_heads / p.n_kv_heads);
  }
  return check_launch("k_attn_partial");
}

}  // namespace

int launch_attn_partial(const AttnParams& p, hipStream_t s) {
  if (p.head_dim == 128) return launch_partial_d<128>(p, s);
  if (p.head_dim == 64) return launch_partial_d<64>(p, s);
  return set_error(BC_ERR_UNSUPPORTED, "attention: head_dim %d", p.head_dim);
}

int launch_attn_reduce(const ReduceParams& p, hipStream_t s) {
  k_attn_reduce<<<dim3(p.n_heads), dim3(kAttnThreads), 0, s>>>(p);
  return check_launch("k_attn_reduce");
}

}  // namespace bc

using namespace bc;

extern "C" int bc_attn_default_splits(int n_sel, int n_kv_heads) {
  if (n_sel <= 0 || n_kv_heads <= 0) return 1;
  // about 1024 work-groups at long context, at least 64 listed tokens each
  int by_len = ceil_div(n_sel, 64);
  int by_fill = 1024 / n_kv_heads;
  if (by_fill < 1) by_fill = 1;
  int s = by_len < by_fill ? by_len : by_fill;
  return s < 1 ? 1 : s;
}

extern "C" int bc_splitk_attn_partial(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                      int n_cap, const int32_t* idx, int n_sel, int n_heads, int n_kv_heads,
                                      int head_dim, int n_splits, float scale, float* m, float* l, float* o,
                                      void* stream) {
  if (!q || !k_cache || !v_cache || !m || !l || !o)
    return set_error(BC_ERR_INVALID, "bc_splitk_attn_partial: NULL pointer");
  if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return set_error(BC_ERR_INVALID, "bc_splitk_attn_partial: heads %d / %d", n_heads, n_kv_heads);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (!valid_group(n_heads / n_kv_heads)) return set_error(BC_ERR_UNSUPPORTED, "group %d", n_heads / n_kv_heads);
  if (n_sel < 0 || n_cap <= 0 || (idx == nullptr && n_sel > n_cap))
    return set_error(BC_ERR_INVALID, "bc_splitk_attn_partial: n_sel=%d n_cap=%d", n_sel, n_cap);
  if (n_splits < 1 || n_splits > 4096)
    return set_error(BC_ERR_INVALID, "bc_splitk_attn_partial: n_splits=%d", n_splits);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 15)
    return set_error(BC_ERR_INVALID, "bc_splitk_attn_partial: q/K/V must be 16-byte aligned");
  AttnParams p{};
  p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.n_cap = n_cap; p.idx = idx; p.n_sel = n_sel;
  p.n_heads = n_heads; p.n_kv_heads = n_kv_heads; p.head_dim = head_dim; p.n_splits = n_splits;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.m = m; p.l = l; p.o = o;
  return launch_attn_partial(p, static_cast<hipStream_t>(stream));
}

extern "C" int bc_splitk_reduce(const float* m, const float* l, const float* o, int n_heads, int n_splits,
                                int head_dim, uint16_t* out, void* stream) {
  if (!m || !l || !o || !out) return set_error(BC_ERR_INVALID, "bc_splitk_reduce: NULL pointer");
  if (n_heads <= 0 || n_splits < 1 || n_splits > 4096)
    return set_error(BC_ERR_INVALID, "bc_splitk_reduce: n_heads=%d n_splits=%d", n_heads, n_splits);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  ReduceParams p{};
  p.m = m; p.l = l; p.o = o; p.n_heads = n_heads; p.n_splits = n_splits; p.head_dim = head_dim;
  p.out = out;
  return launch_attn_reduce(p, static_cast<hipStream_t>(stream));
}
