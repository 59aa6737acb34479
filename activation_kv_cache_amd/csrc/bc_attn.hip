// bc_attn.hip -- split-K grouped-query decode attention for gfx950.
//
// README "Overview": dense and sparse modes read their caches through the
// same split-K attention kernel, so the dense baseline stays fixed.  Here the
// dense mode is the same kernel with idx == NULL.
//
// Partial pass: one work-group per (split, KV head).  A key (value) row is
// head_dim bf16 = 256 B at head_dim 128; a group of 8 lanes holds one row,
// lane r the dims [8r, 8r+8) and [64+8r, 64+8r+8) (two 16-byte loads, each
// covering 128 contiguous bytes of the row across the group), so one wave
// load instruction reads 8 rows.  A wave iteration takes 2 rows per group.
// The G query heads of the KV head live in registers as bf16 pairs; q.k uses
// v_dot2 (bf16 pairs into fp32) and a 3-step DPP sum over the group.  The
// softmax weights are rounded to bf16 and paired over the two rows, so p.v is
// again v_dot2 with fp32 accumulation (the pairs of value rows are formed
// with v_perm); the weight sum l adds the same rounded weights.  Each lane
// group keeps its own online-softmax state and only rescales when the
// running max grows by more than 8 in log2 units.  States are merged across
// the wave with shuffles and across the 4 waves through LDS.  In index mode
// the split's slice of the index list is staged in LDS.
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
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kIdxChunk = 1024;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int G>
struct AttnSmem {
  uint16_t q[G][D];
  float o[kAttnWaves][G][D];
  float m[kAttnWaves][G];
  float l[kAttnWaves][G];
  int32_t idx[kIdxChunk];
};

// Online-softmax state of one lane group: running max m (raw q.k units),
// sum l of the (bf16-rounded) weights, and o over the lane's 16 dims.
template <int G>
struct AttnState {
  float m[G], l[G], o[G][16];
  float mx[G];   // true max of the logits seen (m may lag it by up to tau)
};

// K and V of the two rows a lane group takes in one wave iteration.
struct AttnRows {
  uint4 ka[2], kb[2], va[2], vb[2];
};

// Rows base + u*TPL + sub (u = 0, 1) of the chunk [c0, c1); positions past
// c1 read row c1-1 again (their weight is masked to zero).  Lane r of a row
// group loads dims [8r, 8r+8) and [D/2 + 8r, D/2 + 8r + 8).
template <int D>
__device__ __forceinline__ void attn_load(const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg,
                                          const int32_t* sidx, int base, int c0, int c1, int sub, AttnRows& rw) {
  constexpr int LPT = D / 16;
  constexpr int TPL = kWave / LPT;
  constexpr int HALF = D / 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pos = base + u * TPL + sub;
    const int pc = pos < c1 ? pos : c1 - 1;
    const int t = sidx ? sidx[pc - c0] : pc;
    const size_t off = size_t(t) * D;
    rw.ka[u] = *reinterpret_cast<const uint4*>(Kg + off);
    rw.kb[u] = *reinterpret_cast<const uint4*>(Kg + off + HALF);
    rw.va[u] = *reinterpret_cast<const uint4*>(Vg + off);
    rw.vb[u] = *reinterpret_cast<const uint4*>(Vg + off + HALF);
  }
}

// Online-softmax update of one lane group with its two rows.  q comes from
// LDS ([G][D] bf16; lane r reads its 16 dims of every head).
template <int D, int G, bool MASKED>
__device__ __forceinline__ void attn_compute(const AttnRows& rw, const uint16_t* sq, int base, int c1, int sub, int r,
                                             float c, float tau, AttnState<G>& st) {
  constexpr int LPT = D / 16;
  constexpr int TPL = kWave / LPT;
  constexpr int HALF = D / 2;
  bool valid[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) valid[u] = !MASKED || base + u * TPL + sub < c1;
  float a[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4 q0 = *reinterpret_cast<const uint4*>(sq + j * D + 8 * r);
    const uint4 q1 = *reinterpret_cast<const uint4*>(sq + j * D + HALF + 8 * r);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc = dot2(q0.x, rw.ka[u].x, 0.f);
      acc = dot2(q0.y, rw.ka[u].y, acc);
      acc = dot2(q0.z, rw.ka[u].z, acc);
      acc = dot2(q0.w, rw.ka[u].w, acc);
      acc = dot2(q1.x, rw.kb[u].x, acc);
      acc = dot2(q1.y, rw.kb[u].y, acc);
      acc = dot2(q1.z, rw.kb[u].z, acc);
      acc = dot2(q1.w, rw.kb[u].w, acc);
      acc = group_sum<LPT>(acc);
      a[j][u] = (MASKED && !valid[u]) ? -INFINITY : acc;
    }
  }
  // lazy rescaling: the running max only moves when a new logit exceeds it
  // by more than tau (weights stay below 2^8 in between)
  bool need[G];
  bool any_need = false;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float mt = fmaxf(a[j][0], a[j][1]);
    need[j] = mt > st.m[j] + tau;
    any_need |= need[j];
    st.mx[j] = fmaxf(st.mx[j], mt);
  }
  if (__any(any_need)) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mt = fmaxf(a[j][0], a[j][1]);
      const float mn = need[j] ? mt : st.m[j];
      const float alpha = need[j] ? (st.m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m[j] - mn) * c)) : 1.f;
      st.l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[j][e] *= alpha;
      st.m[j] = mn;
    }
  }
  // value pairs (row 0, row 1) per dim, shared by every head of the group
  uint32_t vp[16];
  {
    const uint32_t w0[8] = {rw.va[0].x, rw.va[0].y, rw.va[0].z, rw.va[0].w,
                            rw.vb[0].x, rw.vb[0].y, rw.vb[0].z, rw.vb[0].w};
    const uint32_t w1[8] = {rw.va[1].x, rw.va[1].y, rw.va[1].z, rw.va[1].w,
                            rw.vb[1].x, rw.vb[1].y, rw.vb[1].z, rw.vb[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vp[2 * i] = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);
      vp[2 * i + 1] = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float mc = st.m[j] == -INFINITY ? 0.f : st.m[j] * c;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(a[j][0], c, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(a[j][1], c, -mc));
    const uint32_t pk = pack_bf16x2(p0, p1);
    st.l[j] += bf16_lo(pk) + bf16_hi(pk);
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[j][e] = dot2(pk, vp[e], st.o[j][e]);
  }
}

// Merge state b into a (same lane dims).
template <int G>
__device__ __forceinline__ void attn_merge(AttnState<G>& a, const AttnState<G>& b, float c) {
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float M = fmaxf(a.m[j], b.m[j]);
    const float wa = a.m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((a.m[j] - M) * c);
    const float wb = b.m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((b.m[j] - M) * c);
    a.l[j] = a.l[j] * wa + b.l[j] * wb;
#pragma unroll
    for (int e = 0; e < 16; ++e) a.o[j][e] = a.o[j][e] * wa + b.o[j][e] * wb;
    a.m[j] = M;
  }
}

template <int D, int G>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(const AttnParams p) {
  constexpr int LPT = D / 16;          // lanes per row
  constexpr int TPL = kWave / LPT;     // rows per wave load
  constexpr int TPI = 2 * TPL;         // rows per wave iteration
  constexpr int HALF = D / 2;
  __shared__ AttnSmem<D, G> sm;

  const int s = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = wave_lane(), w = wave_id();
  const int sub = lane / LPT, r = lane % LPT;
  const int cn = (p.n_sel + p.n_splits - 1) / p.n_splits;
  const int lo = s * cn;
  const int hi = min(p.n_sel, lo + cn);
  const float c = p.scale_log2;
  const float tau = 8.0f / c;

  for (int i = tid; i < G * D / 8; i += kAttnThreads)
    reinterpret_cast<uint4*>(&sm.q[0][0])[i] = reinterpret_cast<const uint4*>(p.q + size_t(g) * G * D)[i];
  AttnState<G> st;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    st.m[j] = -INFINITY;
    st.mx[j] = -INFINITY;
    st.l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[j][e] = 0.f;
  }
  const uint16_t* Kg = p.k_cache + size_t(g) * p.n_cap * D + 8 * r;
  const uint16_t* Vg = p.v_cache + size_t(g) * p.n_cap * D + 8 * r;
  const int32_t* idxg = p.idx ? p.idx + size_t(g) * p.n_sel : nullptr;

  __syncthreads();
  for (int c0 = lo; c0 < hi; c0 += kIdxChunk) {
    const int c1 = min(hi, c0 + kIdxChunk);
    const int32_t* sidx = nullptr;
    if (idxg) {
      for (int i = tid; i < c1 - c0; i += kAttnThreads) sm.idx[i] = idxg[c0 + i];
      __syncthreads();
      sidx = sm.idx;
    }
    int base = c0 + w * TPI;
    for (; base + TPI <= c1; base += kAttnWaves * TPI) {
      AttnRows rw;
      attn_load<D>(Kg, Vg, sidx, base, c0, c1, sub, rw);
      attn_compute<D, G, false>(rw, &sm.q[0][0], base, c1, sub, r, c, tau, st);
    }
    if (base < c1) {
      AttnRows rw;
      attn_load<D>(Kg, Vg, sidx, base, c0, c1, sub, rw);
      attn_compute<D, G, true>(rw, &sm.q[0][0], base, c1, sub, r, c, tau, st);
    }
    if (idxg) __syncthreads();
  }

  // express every lane state at its true max, then merge the row groups of
  // the wave (lanes with the same r), then the waves
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float alpha = st.m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m[j] - st.mx[j]) * c);
    st.l[j] *= alpha;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[j][e] *= alpha;
    st.m[j] = st.mx[j];
  }
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
    AttnState<G> o;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      o.m[j] = __shfl_xor(st.m[j], off, kWave);
      o.l[j] = __shfl_xor(st.l[j], off, kWave);
#pragma unroll
      for (int e = 0; e < 16; ++e) o.o[j][e] = __shfl_xor(st.o[j][e], off, kWave);
    }
    attn_merge<G>(st, o, c);
  }
  if (sub == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sm.o[w][j][8 * r + e] = st.o[j][e];
        sm.o[w][j][HALF + 8 * r + e] = st.o[j][8 + e];
      }
      if (r == 0) { sm.m[w][j] = st.m[j]; sm.l[w][j] = st.l[j]; }
    }
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += kAttnThreads) {
    const int j = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kAttnWaves; ++q) M = fmaxf(M, sm.m[q][j]);
    float acc = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < kAttnWaves; ++q) {
        const float mq = sm.m[q][j];
        if (mq == -INFINITY) continue;
        const float wq = __builtin_amdgcn_exp2f((mq - M) * c);
        acc += sm.o[q][j][d] * wq;
        lsum += sm.l[q][j] * wq;
      }
    }
    const int jh = g * G + j;
    p.o[(size_t(jh) * p.n_splits + s) * D + d] = acc;
    if (d == 0) {
      p.m[size_t(jh) * p.n_splits + s] = M == -INFINITY ? -INFINITY : M * c * kLn2;
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
  // one long-running work-group per compute unit streams best (256 CUs);
  // at short context at least 64 listed tokens per split
  int by_fill = 256 / n_kv_heads;
  if (by_fill < 1) by_fill = 1;
  const int by_len = ceil_div(n_sel, 64);
  const int s = by_len < by_fill ? by_len : by_fill;
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
