// bc_attn.hip -- split-K grouped-query decode attention for gfx950.
//
// README "Overview": one split-K attention kernel serves the dense mode and
// every sparse mode, which keeps the dense reference from moving with the
// mode.  Here the dense mode is the same kernel with idx == NULL.
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

#include "bc_clock.hpp"
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
static_assert(kAttnMaxCand == 8 * kAttnThreads, "prologue block ranking: 8 candidate keys per thread");
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kIdxChunk = 1024;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, nearest even
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int G>
struct AttnSmem {
  static constexpr int NST = kAttnThreads / (D / 16);   // row-group states per work-group
  static constexpr int OSTRIDE = G * D + 4;             // padded: row groups write to different banks
  uint16_t q[G][D];
  uint16_t knew[D];   // the current token's k, v (appending work-group)
  uint16_t vnew[D];
  int32_t blk[kAttnMaxRanks];   // L_SCORES: candidate of each block rank this split reads
  union {
    alignas(16) float st_o[NST * OSTRIDE];   // row-group states (after the main loop)
    Topk32Smem<kAttnThreads> tk;             // block selection (prologue)
  };
  alignas(16) float st_m[G][NST];
  alignas(16) float st_mx[G][NST];
  alignas(16) float st_l[G][NST];
  alignas(16) float wt[G][NST];
  float M[G];
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

// A 16-byte non-temporal load: K and V rows are read once per step, so they
// should not displace the small vectors the kernels share in the caches.
__device__ __forceinline__ uint4 load_nt(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Rows of list positions base + u*TPL + sub (u = 0, 1), below c1; positions
// past c1 read the row of c1-1 again (their weight is masked to zero).
// tok maps a list position to its token.  Lane r of a row group loads dims
// [8r, 8r+8) and [D/2 + 8r, D/2 + 8r + 8).
template <int D, typename TokFn>
__device__ __forceinline__ void attn_load(const uint16_t* __restrict__ Kg, const uint16_t* __restrict__ Vg, TokFn tok,
                                          int base, int c1, int sub, AttnRows& rw) {
  constexpr int LPT = D / 16;
  constexpr int TPL = kWave / LPT;
  constexpr int HALF = D / 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pos = base + u * TPL + sub;
    const int pc = pos < c1 ? pos : c1 - 1;
    const int t = tok(pc);
    const size_t off = size_t(t) * D;
    rw.ka[u] = load_nt(Kg + off);
    rw.kb[u] = load_nt(Kg + off + HALF);
    rw.va[u] = load_nt(Vg + off);
    rw.vb[u] = load_nt(Vg + off + HALF);
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

// Block ranks [r_lo, r_hi) of the exact top-k_blk of n block scores:
// blk[rank - r_lo] = candidate index.  PM keys per thread (n <= NT * PM).
template <int NT, int PM>
__device__ void select_block_ranks(const float* sc, int n, int k_blk, int r_lo, int r_hi, int32_t* blk,
                                   Topk32Smem<NT>& tk) {
  uint32_t key[PM];
  const int P = load_score_keys<NT, PM>(sc, n, key, tk.hist);
  const int tid = threadIdx.x;
  auto emit = [&](int rel, int e) { blk[rel] = tid * P + e; };
  block_topk32<NT, PM>(key, P, n, k_blk, r_lo, r_hi, emit, tk);
}

template <int D, int G, int QM, int LM>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(const AttnParams p) {
  constexpr int LPT = D / 16;          // lanes per row
  constexpr int TPL = kWave / LPT;     // rows per wave load
  constexpr int TPI = 2 * TPL;         // rows per wave iteration
  constexpr int STEP = kAttnWaves * TPI;
  constexpr int HALF = D / 2;
  __shared__ AttnSmem<D, G> sm;
  // phase ends (a build with phase clocks only): [3] q (and the list's
  // block ranks) ready after the prologue's barrier, [12] the first wave's
  // rows done, [5] every wave's rows done (the merge's first barrier), [6]
  // merge weights ready
  PhaseClock clk;
  clk.begin();

  const int s = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, lane = wave_lane(), w = wave_id();
  const int sub = lane / LPT, r = lane % LPT;
  const int cn = (p.n_sel + p.n_splits - 1) / p.n_splits;
  const int lo = s * cn;
  const int hi = min(p.n_sel, lo + cn);
  const float c = p.scale_log2;
  const float tau = 8.0f / c;
  // the work-group holding the current token attends to it from LDS, not
  // from the cache slot it writes
  const bool appends = QM == Q_PARTIAL && lo <= p.pos && p.pos < hi;
  const int hi_main = appends ? p.pos : hi;

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

  // q (and for the appending work-group the current token's k, v) from the
  // qkv GEMV chunk partials: their loads are issued first, since memory
  // counters retire in order and the other loads below are not needed as soon
  constexpr int QPT = (G * HALF + kAttnThreads - 1) / kAttnThreads;
  Chunk8 cqa[QPT], cqb[QPT], cka, ckb, cvv;
  const int kcol = p.n_heads * D + g * D, vcol = (p.n_heads + p.n_kv_heads) * D + g * D;
  if constexpr (QM == Q_PARTIAL) {
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = min(tid + u * kAttnThreads, G * HALF - 1);
      const int col = (g * G + e / HALF) * D + e % HALF;
      chunk_load(cqa[u], p.qkv_partial, p.qkv_splits, p.qkv_out, col);
      chunk_load(cqb[u], p.qkv_partial, p.qkv_splits, p.qkv_out, col + HALF);
    }
    if (appends) {
      const int ih = min(tid, HALF - 1), id = min(tid, D - 1);
      chunk_load(cka, p.qkv_partial, p.qkv_splits, p.qkv_out, kcol + ih);
      chunk_load(ckb, p.qkv_partial, p.qkv_splits, p.qkv_out, kcol + ih + HALF);
      chunk_load(cvv, p.qkv_partial, p.qkv_splits, p.qkv_out, vcol + id);
    }
  }
  // the rotary cos/sin of the thread's pairs: the table is a kernel argument
  // indexed per lane, so these are memory loads, issued before the K/V rows
  // (loads retire in order: issued later, forming q would wait for the rows)
  float rc[QPT], rsn[QPT];
  if constexpr (QM == Q_PARTIAL) {
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int i = min(tid + u * kAttnThreads, G * HALF - 1) % HALF;
      rc[u] = p.rope.c[i];
      rsn[u] = p.rope.s[i];
    }
  }

  // the appending work-group refreshes the (min, max) summary of the
  // current token's block; the block's older rows are loaded now and used
  // at the end, so their latency hides under the main loop
  const bool refresh = QM == Q_PARTIAL && appends && p.summary != nullptr && tid < HALF;
  const int blk = p.pos / 16;
  // two dims per lane, one 32-bit word per row: a full register each, which
  // the compiler keeps as loaded (16-bit values it repacks in pairs right
  // after the loads, and then waits for them before the K/V row loads)
  uint32_t srow[16];
  if (refresh) {
    const uint32_t* kc = reinterpret_cast<const uint32_t*>(p.k_cache + size_t(g) * p.n_cap * D) + tid;
    // rows from pos on are replaced by the new row later; their loads read
    // an older row (clamped index, no branches)
#pragma unroll
    for (int t = 0; t < 16; ++t) srow[t] = kc[size_t(max(0, min(blk * 16 + t, p.pos - 1))) * HALF];
  }

  // dense list: the first rows are known before q, so they go in flight now
  AttnRows rw;
  int base = lo + w * TPI;
  auto tok_dense = [](int pc) { return pc; };
  // the rows of list positions [base, c1) in steps of STEP, rw already
  // holding those of base (< c1); software-pipelined: a wave's next rows are
  // in flight while it computes the current ones (two row buffers taken in
  // turn; a load past c1 reads row c1-1 again and is never used)
  auto stream_rows = [&](auto tok, int c1) {
    AttnRows nx;
    attn_load<D>(Kg, Vg, tok, base + STEP, c1, sub, nx);
    for (;;) {
      attn_compute<D, G, true>(rw, &sm.q[0][0], base, c1, sub, r, c, tau, st);
      base += STEP;
      if (base >= c1) break;
      attn_load<D>(Kg, Vg, tok, base + STEP, c1, sub, rw);
      attn_compute<D, G, true>(nx, &sm.q[0][0], base, c1, sub, r, c, tau, st);
      base += STEP;
      if (base >= c1) break;
      attn_load<D>(Kg, Vg, tok, base + STEP, c1, sub, nx);
    }
  };
  if constexpr (LM == L_DENSE) {
    if (base < hi_main) attn_load<D>(Kg, Vg, tok_dense, base, hi_main, sub, rw);
  }

  // scored list: the block ranks [r_lo, r_hi) this split's slice reads
  int r_lo = 0, r_hi = 0;
  if constexpr (LM == L_SCORES) {
    const int S0 = p.bud.sinks, KB = p.bud.k_blk;
    if (KB > 0 && hi > S0 && lo < S0 + 16 * KB) {
      r_lo = lo > S0 ? (lo - S0) / 16 : 0;
      r_hi = min(KB, (hi - S0 + 15) / 16);
    }
    if (r_lo < r_hi && p.blk) {   // ranks from the selection kernel
      const int32_t* bg = p.blk + size_t(g) * KB + r_lo;
      for (int i = tid; i < r_hi - r_lo; i += kAttnThreads) sm.blk[i] = bg[i];
    } else if (r_lo < r_hi) {   // uniform over the work-group
      const int n = p.bud.n_cand;
      const float* sc = p.scores + size_t(g) * p.scores_stride;
      // n <= kAttnMaxCand: 8 keys per thread (more candidates are ranked by
      // their own kernel, which measured faster)
      select_block_ranks<kAttnThreads, kAttnMaxCand / kAttnThreads>(sc, n, KB, r_lo, r_hi, sm.blk, sm.tk);
    }
  }

  if constexpr (QM == Q_GLOBAL) {
    for (int i = tid; i < G * D / 8; i += kAttnThreads)
      reinterpret_cast<uint4*>(&sm.q[0][0])[i] = reinterpret_cast<const uint4*>(p.q + size_t(g) * G * D)[i];
  } else {
    // rotary pairs (i, i + D/2) of the group's heads, chunks added in chunk
    // order, rounded to bf16
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = tid + u * kAttnThreads;
      if (e >= G * HALF) continue;
      const int j = e / HALF, i = e % HALF;
      const float qa = chunk_total(cqa[u], p.qkv_splits);
      const float qb = chunk_total(cqb[u], p.qkv_splits);
      const float cs = rc[u], sn = rsn[u];
      const uint16_t q0 = f32_to_bf16(qa * cs - qb * sn), q1 = f32_to_bf16(qb * cs + qa * sn);
      sm.q[j][i] = q0;
      sm.q[j][i + HALF] = q1;
      if (s == 0 && p.q_out) {
        p.q_out[size_t(g * G + j) * D + i] = q0;
        p.q_out[size_t(g * G + j) * D + i + HALF] = q1;
      }
    }
    if (appends) {
      uint16_t* kr = p.k_cache + (size_t(g) * p.n_cap + p.pos) * D;
      uint16_t* vr = p.v_cache + (size_t(g) * p.n_cap + p.pos) * D;
      if (tid < HALF) {
        const float ka = chunk_total(cka, p.qkv_splits);
        const float kb = chunk_total(ckb, p.qkv_splits);
        // pair tid: the pair of q element tid as well (tid < D/2 <= G*D/2)
        const float cs = rc[0], sn = rsn[0];
        const uint16_t k0 = f32_to_bf16(ka * cs - kb * sn), k1 = f32_to_bf16(kb * cs + ka * sn);
        sm.knew[tid] = k0;
        sm.knew[tid + HALF] = k1;
        kr[tid] = k0;
        kr[tid + HALF] = k1;
      }
      if (tid < D) {
        const uint16_t v0 = f32_to_bf16(chunk_total(cvv, p.qkv_splits));
        sm.vnew[tid] = v0;
        vr[tid] = v0;
      }
    }
  }
  __syncthreads();
  clk.stamp(3);

  if constexpr (LM != L_IDX) {
    // one pass over the split's list positions [lo, hi_main): the dense list
    // is tokens themselves; a scored list maps a position to its token from
    // the budget and the selected block ranks (sinks | blocks | window), so
    // nothing is staged and the row loads stay pipelined across the split
    const int S0 = p.bud.sinks, nb0 = p.bud.sinks + 16 * p.bud.k_blk;
    const int rmax = max(r_hi - r_lo - 1, 0);
    auto tok_scored = [&](int pc) -> int {
      const int q = pc - S0;
      const int ri = min(max((q >> 4) - r_lo, 0), rmax);
      const int tb = 16 * (p.bud.b_lo + sm.blk[ri]) + (q & 15);
      const int tw = p.n_ctx - p.bud.window + (pc - nb0);
      return pc < S0 ? pc : (pc < nb0 ? tb : tw);
    };
    auto run = [&](auto tok) {
      const int c1 = hi_main;
      if (base >= c1) return;
      if constexpr (LM == L_SCORES) attn_load<D>(Kg, Vg, tok, base, c1, sub, rw);
      stream_rows(tok, c1);
    };
    if constexpr (LM == L_DENSE) {
      run(tok_dense);
    } else {
      if (p.idx_out) {
        int32_t* io = p.idx_out + size_t(g) * p.n_sel;
        for (int i = lo + tid; i < hi; i += kAttnThreads) io[i] = tok_scored(i);
      }
      run(tok_scored);
    }
  } else {
    const int32_t* idxg = p.idx + size_t(g) * p.n_sel;
    for (int c0 = lo; c0 < hi; c0 += kIdxChunk) {
      const int c1 = min(hi, c0 + kIdxChunk);
      // the chunk's tokens from the index list (4 positions per thread; the
      // loads are all issued before the stores)
      static_assert(kIdxChunk == 4 * kAttnThreads, "chunk of 4 positions per thread");
      int32_t tk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) tk[u] = tid + u * kAttnThreads < c1 - c0 ? idxg[c0 + tid + u * kAttnThreads] : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (tid + u * kAttnThreads < c1 - c0) sm.idx[tid + u * kAttnThreads] = tk[u];
      __syncthreads();
      auto tok = [&](int pc) -> int { return sm.idx[pc - c0]; };
      base = c0 + w * TPI;
      if (base < c1) {
        attn_load<D>(Kg, Vg, tok, base, c1, sub, rw);
        stream_rows(tok, c1);
      }
      __syncthreads();
    }
  }

  // the current token: wave 0, lane group 0 takes it as its row 0; every
  // other row of that step is masked
  if (appends && w == 0) {
    AttnRows nr;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      nr.ka[u] = *reinterpret_cast<const uint4*>(sm.knew + 8 * r);
      nr.kb[u] = *reinterpret_cast<const uint4*>(sm.knew + HALF + 8 * r);
      nr.va[u] = *reinterpret_cast<const uint4*>(sm.vnew + 8 * r);
      nr.vb[u] = *reinterpret_cast<const uint4*>(sm.vnew + HALF + 8 * r);
    }
    attn_compute<D, G, true>(nr, &sm.q[0][0], 0, 1, sub, r, c, tau, st);
  }

  clk.stamp_after(12, st.l[0] + st.o[0][15]);
  // merge the row groups' states in LDS: every row group writes its lazy
  // state (m, l, o) and its true max; the weight of state k for head j is
  // 2^((m_k - M_j) c) with M_j the largest true max, and each output dim is
  // the weighted sum over the states in state order
  {
    using SM = AttnSmem<D, G>;
    constexpr int NSUB = kWave / LPT;
    const int k = w * NSUB + sub;
    float* so = sm.st_o + k * SM::OSTRIDE;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float4* d0 = reinterpret_cast<float4*>(so + j * D + 8 * r);
      float4* d1 = reinterpret_cast<float4*>(so + j * D + HALF + 8 * r);
      d0[0] = make_float4(st.o[j][0], st.o[j][1], st.o[j][2], st.o[j][3]);
      d0[1] = make_float4(st.o[j][4], st.o[j][5], st.o[j][6], st.o[j][7]);
      d1[0] = make_float4(st.o[j][8], st.o[j][9], st.o[j][10], st.o[j][11]);
      d1[1] = make_float4(st.o[j][12], st.o[j][13], st.o[j][14], st.o[j][15]);
      if (r == 0) {
        sm.st_m[j][k] = st.m[j];
        sm.st_mx[j][k] = st.mx[j];
        sm.st_l[j][k] = st.l[j];
      }
    }
    __syncthreads();
    clk.stamp(5);
    static_assert(SM::NST % 4 == 0, "states in float4 groups");
    for (int e = tid; e < G * SM::NST; e += kAttnThreads) {
      const int j = e / SM::NST, kk = e % SM::NST;
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < SM::NST; q += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&sm.st_mx[j][q]);
        M = fmaxf(M, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
      }
      const float mk = sm.st_m[j][kk];
      sm.wt[j][kk] = mk == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mk - M) * c);
      if (kk == 0) sm.M[j] = M;
    }
    __syncthreads();
    clk.stamp(6);
    // two adjacent dims per thread (64-bit LDS reads), weights four at a time
    for (int e = 2 * tid; e < G * D; e += 2 * kAttnThreads) {
      const int j = e / D, d = e % D;
      float ax = 0.f, ay = 0.f;
#pragma unroll
      for (int q = 0; q < SM::NST; q += 4) {
        const float4 wv = *reinterpret_cast<const float4*>(&sm.wt[j][q]);
        const float wq[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float2 ov = *reinterpret_cast<const float2*>(&sm.st_o[(q + u) * SM::OSTRIDE + j * D + d]);
          ax += ov.x * wq[u];
          ay += ov.y * wq[u];
        }
      }
      const int jh = g * G + j;
      *reinterpret_cast<float2*>(&p.o[(size_t(jh) * p.n_splits + s) * D + d]) = make_float2(ax, ay);
      if (d == 0) {
        float lsum = 0.f;
#pragma unroll
        for (int q = 0; q < SM::NST; q += 4) {
          const float4 lv = *reinterpret_cast<const float4*>(&sm.st_l[j][q]);
          const float4 wv = *reinterpret_cast<const float4*>(&sm.wt[j][q]);
          lsum += lv.x * wv.x;
          lsum += lv.y * wv.y;
          lsum += lv.z * wv.z;
          lsum += lv.w * wv.w;
        }
        const float M = sm.M[j];
        p.m[size_t(jh) * p.n_splits + s] = M == -INFINITY ? -INFINITY : M * c * kLn2;
        p.l[size_t(jh) * p.n_splits + s] = lsum;
      }
    }
  }
  if (refresh) {
    // dims 2*tid and 2*tid + 1, (min, max) each: the new row first, then
    // rows 16*blk.. in order (rows from pos on are the new row); an equal
    // value never replaces an earlier one
    uint32_t mm[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t nb = sm.knew[2 * tid + h];
      uint16_t bmn = nb, bmx = nb;
      float mn = bf16_to_f32(nb), mx = mn;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const uint16_t u = blk * 16 + t < p.pos ? uint16_t(srow[t] >> (16 * h)) : nb;
        const float f = bf16_to_f32(u);
        if (f < mn) { mn = f; bmn = u; }
        if (f > mx) { mx = f; bmx = u; }
      }
      mm[h] = uint32_t(bmn) | (uint32_t(bmx) << 16);
    }
    uint16_t* sp = p.summary + ((size_t(g) * (p.n_cap / 16) + blk) * D + 2 * tid) * 2;
    *reinterpret_cast<uint2*>(sp) = make_uint2(mm[0], mm[1]);
  }
  clk.end(p.clk, size_t(g) * gridDim.x + s);
}

// One work-group per query head.  M and the weights w_s = e^(m_s - M) are
// computed once into LDS; the weighted sums over splits are split between
// thread groups (fixed halves) and combined in a fixed order.
constexpr int kReduceMaxSplits = 4096;

// Up to kAttnFoldMaxSplits splits every load goes out before any arithmetic
// (m and l of split tid, the thread's o values): one memory round trip
// instead of one per phase.  The arithmetic is the same in either case.
constexpr int kReducePre = kAttnFoldMaxSplits / 2;   // o values per thread (head_dim >= 64: >= 2 groups)

__global__ __launch_bounds__(kAttnThreads) void k_attn_reduce(const ReduceParams p) {
  static_assert(kAttnThreads == kCombineThreads, "one thread per den term slot of the combine order");
  static_assert(kAttnFoldMaxSplits <= kWave, "preloaded m and l sit in wave 0");
  __shared__ float wts[kReduceMaxSplits];
  __shared__ float part[kAttnThreads];
  __shared__ float red[kAttnThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = blockIdx.x;
  const int D = p.head_dim, S = p.n_splits;
  const float* mj = p.m + size_t(j) * S;
  const float* lj = p.l + size_t(j) * S;
  const int groups = kAttnThreads / D;          // 2 at head_dim 128, 4 at 64
  const int grp = tid / D, d = tid % D;
  const int per = (S + groups - 1) / groups;
  const int s0 = min(S, grp * per), s1 = min(S, s0 + per);
  const float* oj = p.o + size_t(j) * S * D + d;
  const bool pre = S <= kAttnFoldMaxSplits && per <= kReducePre;   // uniform
  float mp = -INFINITY, lp = 0.f;
  float ov[kReducePre];
  if (pre) {
    if (tid < S) {
      mp = mj[tid];
      lp = lj[tid];
    }
    // clamped, unconditional loads (splits past the group's end are dropped below)
#pragma unroll
    for (int i = 0; i < kReducePre; ++i) ov[i] = oj[size_t(min(s0 + i, S - 1)) * D];
  }
  float mx = -INFINITY;
  if (pre)
    mx = mp;
  else
    for (int s = tid; s < S; s += kAttnThreads) mx = fmaxf(mx, mj[s]);
  mx = wave_max_f32(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < kAttnThreads / kWave; ++i) M = fmaxf(M, red[i]);
  __syncthreads();
  float den = 0.f;
  if (pre) {
    if (tid < S) {
      const float wt = combine_weight(mp, M);
      wts[tid] = wt;
      den = fmaf(wt, lp, den);
    }
  } else {
    for (int s = tid; s < S; s += kAttnThreads) {
      const float wt = combine_weight(mj[s], M);
      wts[s] = wt;
      den = fmaf(wt, lj[s], den);
    }
  }
  den = combine_wave_sum(den);
  if (lane == 0) red[w] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int i = 0; i < kAttnThreads / kWave; ++i) den += red[i];
  float num;
  if (pre) {
    // combine_group over registers, in split order
    num = 0.f;
#pragma unroll
    for (int i = 0; i < kReducePre; ++i) {
      const float nx = fmaf(ov[i], wts[min(s0 + i, S - 1)], num);
      num = s0 + i < s1 ? nx : num;
    }
  } else {
    num = combine_group(s0, s1, [&](int s) { return oj[size_t(s) * D]; }, [&](int s) { return wts[s]; });
  }
  part[tid] = num;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int g = 0; g < groups; ++g) t += part[g * D + tid];
    p.out[size_t(j) * D + tid] = f32_to_bf16(den > 0.f ? t / den : 0.f);
  }
}

template <int D, int QM, int LM>
int launch_partial_dql(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.n_splits, p.n_kv_heads), block(kAttnThreads);
  switch (p.n_heads / p.n_kv_heads) {
    case 1: k_attn_partial<D, 1, QM, LM><<<grid, block, 0, s>>>(p); break;
    case 2: k_attn_partial<D, 2, QM, LM><<<grid, block, 0, s>>>(p); break;
    case 4: k_attn_partial<D, 4, QM, LM><<<grid, block, 0, s>>>(p); break;
    case 8: k_attn_partial<D, 8, QM, LM><<<grid, block, 0, s>>>(p); break;
    default: return set_error(BC_ERR_UNSUPPORTED, "attention: group size %d", p.n_heads / p.n_kv_heads);
  }
  return check_launch("k_attn_partial");
}

template <int D>
int launch_partial_d(int q_mode, int list_mode, const AttnParams& p, hipStream_t s) {
  if (q_mode == Q_PARTIAL) {
    if (list_mode != L_DENSE) return set_error(BC_ERR_INVALID, "attention: q from partials needs the dense list");
    return launch_partial_dql<D, Q_PARTIAL, L_DENSE>(p, s);
  }
  if (list_mode == L_IDX) return launch_partial_dql<D, Q_GLOBAL, L_IDX>(p, s);
  if (list_mode == L_SCORES) return launch_partial_dql<D, Q_GLOBAL, L_SCORES>(p, s);
  return launch_partial_dql<D, Q_GLOBAL, L_DENSE>(p, s);
}

}  // namespace

// Largest number of block ranks a split of a scored list reads.
static int scored_ranks_per_split(int n_sel, int n_splits) {
  const int cn = (n_sel + n_splits - 1) / n_splits;
  return cn / 16 + 2;
}

bool attn_scored_list_ok(const bc_kv_budget_info& bud, int n_splits) {
  return scored_ranks_per_split(bud.t_sel, n_splits) <= kAttnMaxRanks;
}

bool attn_prologue_select_ok(const bc_kv_budget_info& bud) { return bud.n_cand <= kAttnMaxCand; }

int launch_attn_partial(int q_mode, int list_mode, const AttnParams& p_in, hipStream_t s) {
  AttnParams p = p_in;
  p.clk = clock_take(size_t(p.n_splits) * p.n_kv_heads, CLOCK_ATTN, q_mode | (list_mode << 8), p.n_sel, p.n_splits,
                     p.n_kv_heads);
  if (list_mode == L_IDX && p.idx == nullptr) return set_error(BC_ERR_INVALID, "attention: NULL index list");
  if (q_mode == Q_PARTIAL && (p.qkv_splits < 1 || p.qkv_splits > kQkvMaxChunks))
    return set_error(BC_ERR_INVALID, "attention: %d q/k/v chunks (1..%d)", p.qkv_splits, kQkvMaxChunks);
  if (list_mode == L_SCORES &&
      (!attn_scored_list_ok(p.bud, p.n_splits) || p.n_sel != p.bud.t_sel ||
       (!p.blk && p.bud.k_blk > 0 && (!p.scores || p.bud.n_cand > kAttnMaxCand))))
    return set_error(BC_ERR_INVALID, "attention: scored list out of range");
  if (p.head_dim == 128) return launch_partial_d<128>(q_mode, list_mode, p, s);
  if (p.head_dim == 64) return launch_partial_d<64>(q_mode, list_mode, p, s);
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
  p.q = q; p.k_cache = const_cast<uint16_t*>(k_cache); p.v_cache = const_cast<uint16_t*>(v_cache);
  p.n_cap = n_cap; p.idx = idx; p.n_sel = n_sel;
  p.n_heads = n_heads; p.n_kv_heads = n_kv_heads; p.head_dim = head_dim; p.n_splits = n_splits;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.m = m; p.l = l; p.o = o;
  return launch_attn_partial(Q_GLOBAL, idx ? L_IDX : L_DENSE, p, static_cast<hipStream_t>(stream));
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
