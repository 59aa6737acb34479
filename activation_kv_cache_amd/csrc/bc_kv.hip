// bc_kv.hip -- attention-scored KV selection for gfx950.
//
// README "What it does in one picture": the selection, scored by attention,
// keeps the first tokens, a share of the older history and the newest tokens.  History is scored
// per 16-token block with an upper bound of the query-key product built from
// the block's per-dimension key minima and maxima (the query-aware block
// bound of Quest, one of the paper's listed ancestors), summed over the
// query heads that share the KV head.
//
// Summary layout: [n_kv_heads][n_cap/16][head_dim][2] bf16, (min, max) per
// dim, so one 16-byte load gives 4 dims of a block.
// Scoring: 32 lanes per block at head_dim 128 (16 at 64), lane p holds dims
// 4p..4p+3 of the group's positive and negative query sums P_d, N_d (each
// an adjacent-pair tree over the heads); the fixed fp32 order is
//   t_d = fma(kmax_d, P_d, kmin_d * N_d),
//   a_p = (t_{4p} + t_{4p+1}) + (t_{4p+2} + t_{4p+3}),
//   s = adjacent-pair tree over p,
// the last one being the xor-1,2,4,8,16 butterfly over the lanes.  Summed
// over the heads, max(q kmax, q kmin) is kmax P + kmin N (kmax >= kmin), so
// each dim costs one product pair, not one per head.
// Selection (block_topk32, exact; equal scores keep the lower block): in the
// decode layer every attention work-group selects the block ranks of its own
// slice of the list in its prologue; bc_kv_score_select writes the whole
// list sinks | kept blocks' tokens | window with one 1024-thread
// work-group per KV head.
#include <math.h>

#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

constexpr int kScoreThreads = 1024;
// Candidate blocks per scoring work-group: 256, one work-group per CU at
// 128K tokens (8 KV heads); with more candidates than one round of such
// work-groups covers, up to 384 per group (the loads all in registers), so
// that one round still covers them
constexpr int kScoreBlocksPerGroup = 256;
constexpr int kScoreTargetGroups = 256;     // work-groups (over all KV heads) one round holds
constexpr int kSelThreads = 1024;
constexpr int kSelMaxCand = kSelThreads * 32;

// A 16-byte non-temporal load: the summaries are read once per step.
__device__ __forceinline__ uint4 load_nt16(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Scores of the candidate blocks of KV head blockIdx.y (256 per work-group).
// QP: q comes from the qkv GEMV chunk partials (rotary from the host table,
// bf16 rounding); the first work-group of each KV head also stores q,
// appends k, v of the current token at slot pos and refreshes the (min, max)
// summary of block pos/16 (which is then never a candidate).
// NIT wave loads of summaries per lane (a group of at most NIT * 16 waves *
// CPW blocks), all issued before q is formed.
template <int D, int G, bool QP, int NIT>
__global__ __launch_bounds__(kScoreThreads) void k_kv_score(const KvSelectParams p) {
  constexpr int P = D / 4;            // lanes per candidate block
  constexpr int CPW = kWave / P;      // candidate blocks per wave load
  constexpr int HALF = D / 2;
  __shared__ uint16_t sq[G][D];
  __shared__ uint16_t knew[D];
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = wave_lane(), w = wave_id();
  const int cs = lane / P, pp = lane % P;
  const int n_cand = p.bud.n_cand;
  const bool first = QP && blockIdx.x == 0;
  // loads in the order they are needed (memory counters retire in order):
  // the qkv chunk partials (QP), the current block's older rows (first
  // group), then every summary this wave scores
  constexpr int QPT = (G * HALF + kScoreThreads - 1) / kScoreThreads;
  Chunk8 cqa[QPT], cqb[QPT], cka, ckb, cvv;
  const int kcol = p.n_heads * D + g * D, vcol = (p.n_heads + p.n_kv_heads) * D + g * D;
  if constexpr (QP) {
    // only the threads that form q load its partials, so the summary loads
    // of the other waves queue behind none
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = tid + u * kScoreThreads;
      if (e < G * HALF) {
        const int col = (g * G + e / HALF) * D + e % HALF;
        chunk_load(cqa[u], p.qkv_partial, p.qkv_splits, p.qkv_out, col);
        chunk_load(cqb[u], p.qkv_partial, p.qkv_splits, p.qkv_out, col + HALF);
      }
    }
    if (first) {
      const int ih = min(tid, HALF - 1), id = min(tid, D - 1);
      chunk_load(cka, p.qkv_partial, p.qkv_splits, p.qkv_out, kcol + ih);
      chunk_load(ckb, p.qkv_partial, p.qkv_splits, p.qkv_out, kcol + ih + HALF);
      chunk_load(cvv, p.qkv_partial, p.qkv_splits, p.qkv_out, vcol + id);
    }
  }
  // the rotary cos/sin of the thread's pairs: the table is a kernel argument
  // indexed per lane, so these are memory loads, issued before the summaries
  // (loads retire in order: issued later, forming q would wait for them all)
  float rc[QPT], rsn[QPT];
  if constexpr (QP) {
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int i = min(tid + u * kScoreThreads, G * HALF - 1) % HALF;
      rc[u] = p.rope.c[i];
      rsn[u] = p.rope.s[i];
    }
  }
  const int blk = p.pos / 16;
  // two dims per lane, one 32-bit word per row: a full register each, which
  // the compiler keeps as loaded (nothing waits for these loads before their
  // use at the end)
  const bool refresh = first && p.summary && tid < HALF;
  uint32_t srow[16];
  if (refresh) {
    const uint32_t* kc = reinterpret_cast<const uint32_t*>(p.k_cache + size_t(g) * p.n_cap * D) + tid;
    // rows from pos on are replaced by the new row later; their loads read
    // an older row (clamped index, no branches)
#pragma unroll
    for (int t = 0; t < 16; ++t) srow[t] = kc[size_t(max(0, min(blk * 16 + t, p.pos - 1))) * HALF];
  }
  const int cbeg = blockIdx.x * p.score_bpg;
  const int cend = min(n_cand, cbeg + p.score_bpg);
  const uint16_t* sg = p.summary + size_t(g) * p.nb_cap * D * 2;
  uint4 mm[NIT];
  if (p.bud.k_blk > 0) {
    // candidates past the group's end re-read its first block (discarded)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = cbeg + (it * (kScoreThreads / kWave) + w) * CPW + cs;
      const int b = p.bud.b_lo + (c < cend ? c : cbeg);
      mm[it] = load_nt16(sg + (size_t(b) * D + 4 * pp) * 2);
    }
  }

  float qf[G][4];
  if constexpr (QP) {
    // q: rotary pairs, chunks added in chunk order, bf16; the first group
    // also stores q, appends k, v and refreshes the current block's summary
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int e = tid + u * kScoreThreads;
      if (e >= G * HALF) continue;
      const int j = e / HALF, i = e % HALF;
      const float qa = chunk_total(cqa[u], p.qkv_splits);
      const float qb = chunk_total(cqb[u], p.qkv_splits);
      const float c = rc[u], sn = rsn[u];
      const uint16_t q0 = f32_to_bf16(qa * c - qb * sn), q1 = f32_to_bf16(qb * c + qa * sn);
      sq[j][i] = q0;
      sq[j][i + HALF] = q1;
      if (first) {
        p.q_out[size_t(g * G + j) * D + i] = q0;
        p.q_out[size_t(g * G + j) * D + i + HALF] = q1;
      }
    }
    if (first) {
      uint16_t* kr = p.k_cache + (size_t(g) * p.n_cap + p.pos) * D;
      uint16_t* vr = p.v_cache + (size_t(g) * p.n_cap + p.pos) * D;
      if (tid < HALF) {
        const float ka = chunk_total(cka, p.qkv_splits);
        const float kb = chunk_total(ckb, p.qkv_splits);
        // pair tid: the pair of q element tid as well (tid < D/2 <= G*D/2)
        const float c = rc[0], sn = rsn[0];
        const uint16_t k0 = f32_to_bf16(ka * c - kb * sn), k1 = f32_to_bf16(kb * c + ka * sn);
        knew[tid] = k0;
        knew[tid + HALF] = k1;
        kr[tid] = k0;
        kr[tid + HALF] = k1;
      }
      if (tid < D) vr[tid] = f32_to_bf16(chunk_total(cvv, p.qkv_splits));
    }
    __syncthreads();
    if (refresh) {
      // dims 2*tid and 2*tid + 1, (min, max) each: the new row first, then
      // rows 16*blk.. in order (rows from pos on are the new row); an equal
      // value never replaces an earlier one
      uint32_t mm2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t nb = knew[2 * tid + h];
        uint16_t bmn = nb, bmx = nb;
        float mn = bf16_to_f32(nb), mx = mn;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const uint16_t u = blk * 16 + t < p.pos ? uint16_t(srow[t] >> (16 * h)) : nb;
          const float f = bf16_to_f32(u);
          if (f < mn) { mn = f; bmn = u; }
          if (f > mx) { mx = f; bmx = u; }
        }
        mm2[h] = uint32_t(bmn) | (uint32_t(bmx) << 16);
      }
      uint16_t* sp = p.summary + ((size_t(g) * p.nb_cap + blk) * D + 2 * tid) * 2;
      *reinterpret_cast<uint2*>(sp) = make_uint2(mm2[0], mm2[1]);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint2 t = *reinterpret_cast<const uint2*>(&sq[j][4 * pp]);
      qf[j][0] = bf16_lo(t.x); qf[j][1] = bf16_hi(t.x);
      qf[j][2] = bf16_lo(t.y); qf[j][3] = bf16_hi(t.y);
    }
  } else {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint2 t = *reinterpret_cast<const uint2*>(p.q + size_t(g * G + j) * D + 4 * pp);
      qf[j][0] = bf16_lo(t.x); qf[j][1] = bf16_hi(t.x);
      qf[j][2] = bf16_lo(t.y); qf[j][3] = bf16_hi(t.y);
    }
  }
  if (p.bud.k_blk <= 0) return;
  // per dim the group's positive and negative query parts, each an
  // adjacent-pair tree over the heads: sum_j max(q kmax, q kmin) is then
  // kmax * P + kmin * N, one product pair per dim instead of one per head
  float pq[4], nq[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float ps[G], ns[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      ps[j] = qf[j][u] > 0.f ? qf[j][u] : 0.f;
      ns[j] = qf[j][u] > 0.f ? 0.f : qf[j][u];
    }
#pragma unroll
    for (int len = G; len > 1; len >>= 1)
#pragma unroll
      for (int i = 0; i < len / 2; ++i) {
        ps[i] = ps[2 * i] + ps[2 * i + 1];
        ns[i] = ns[2 * i] + ns[2 * i + 1];
      }
    pq[u] = ps[0];
    nq[u] = ns[0];
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = cbeg + (it * (kScoreThreads / kWave) + w) * CPW + cs;
    const bool valid = c < cend;
    const uint4 m4 = mm[it];
    const float mn[4] = {bf16_lo(m4.x), bf16_lo(m4.y), bf16_lo(m4.z), bf16_lo(m4.w)};
    const float mx[4] = {bf16_hi(m4.x), bf16_hi(m4.y), bf16_hi(m4.z), bf16_hi(m4.w)};
    float t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float lo = mn[u] * nq[u];
      t[u] = __builtin_fmaf(mx[u], pq[u], lo);
    }
    float v = (t[0] + t[1]) + (t[2] + t[3]);
    v = v + dpp_f<kDppXor1>(v);
    v = v + dpp_f<kDppXor2>(v);
    v = v + dpp_f<kDppHalfMirror>(v);
    v = v + dpp_f<kDppMirror>(v);
    if constexpr (P == 32) v = v + lane_xor<16>(v);
    if (valid && pp == 0) p.scores[size_t(g) * p.scores_stride + c] = v;
  }
}

// The list of KV head blockIdx.x: sinks, the tokens of the k_blk blocks
// with the highest scores (block_topk32 on order-preserving keys; equal
// scores keep the lower block), the window; ascending.
__global__ __launch_bounds__(kSelThreads) void k_kv_block_select(const KvSelectParams p) {
  __shared__ Topk32Smem<kSelThreads> sm;
  __shared__ uint32_t stage16[kSelThreads * 16];   // coalesced staging of up to 16 keys per thread
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const bc_kv_budget_info bd = p.bud;
  int32_t* out = p.idx_out ? p.idx_out + size_t(g) * bd.t_sel : nullptr;
  int32_t* bout = p.blk_out ? p.blk_out + size_t(g) * bd.k_blk : nullptr;
  if (out) {
    for (int t = tid; t < bd.sinks; t += kSelThreads) out[t] = t;
    for (int t = tid; t < bd.window; t += kSelThreads) out[bd.t_sel - bd.window + t] = p.n_ctx - bd.window + t;
  }
  if (bd.k_blk <= 0) return;
  const int n = bd.n_cand;
  const int b_lo = bd.b_lo, sinks = bd.sinks;
  const float* sc = p.scores + size_t(g) * p.scores_stride;
  auto emit_for = [&](int P) {
    return [=](int rk, int e) {
      const int cand = tid * P + e;
      if (bout) bout[rk] = cand;
      if (out) {
        int32_t* o = out + sinks + 16 * rk;
        const int t0 = 16 * (b_lo + cand);
#pragma unroll
        for (int u = 0; u < 16; ++u) o[u] = t0 + u;
      }
    };
  };
  if (n <= kSelThreads * 8) {
    // up to 8 keys per thread, staged through LDS (coalesced loads)
    uint32_t key[8];
    const int P = load_score_keys<kSelThreads, 8>(sc, n, key, sm.hist);
    block_topk32<kSelThreads, 8>(key, P, n, bd.k_blk, 0, bd.k_blk, emit_for(P), sm);
  } else if (n <= kSelThreads * 16) {
    // up to 16 keys per thread (a context of up to 256K tokens), staged the
    // same way
    uint32_t key[16];
    const int P = load_score_keys<kSelThreads, 16>(sc, n, key, stage16);
    block_topk32<kSelThreads, 16>(key, P, n, bd.k_blk, 0, bd.k_blk, emit_for(P), sm);
  } else {
    const int P = (n + kSelThreads - 1) / kSelThreads;
    uint32_t key[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) key[e] = (e < P && tid * P + e < n) ? float_order_key(sc[size_t(tid) * P + e]) : 0u;
    block_topk32<kSelThreads, 32>(key, P, n, bd.k_blk, 0, bd.k_blk, emit_for(P), sm);
  }
}

// One wave per (block, KV head): per dim the min and max over the block's
// tokens below n_ctx.
// Gather of the selected rows into a compact cache: one 16-byte piece of a
// K or V row per thread; row t of head g of the output is row idx[g][t] of
// the cache (ids clamped to the cache, so a bad id cannot read outside it).
__global__ __launch_bounds__(256) void k_kv_compact(const uint16_t* k_cache, const uint16_t* v_cache, int n_cap,
                                                   int head_dim, const int32_t* idx, int t_sel, uint16_t* k_out,
                                                   uint16_t* v_out, int n_cap_out) {
  const int g = blockIdx.y;
  const int per_row = head_dim / 8;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)t_sel * per_row) return;
  const int t = int(i / per_row), c = int(i % per_row);
  const int src = min(max(idx[size_t(g) * t_sel + t], 0), n_cap - 1);
  const size_t si = (size_t(g) * n_cap + src) * head_dim + 8 * c;
  const size_t di = (size_t(g) * n_cap_out + t) * head_dim + 8 * c;
  *reinterpret_cast<uint4*>(k_out + di) = *reinterpret_cast<const uint4*>(k_cache + si);
  *reinterpret_cast<uint4*>(v_out + di) = *reinterpret_cast<const uint4*>(v_cache + si);
}

__global__ __launch_bounds__(256) void k_build_summary(const uint16_t* k_cache, int n_cap, int head_dim, int n_ctx,
                                                      uint16_t* summary) {
  const int g = blockIdx.y;
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nb = (n_ctx + 15) / 16;
  if (blk >= nb) return;
  const int lane = threadIdx.x & 63;
  const int t0 = blk * 16, t1 = min(n_ctx, t0 + 16);
  for (int d = lane; d < head_dim; d += kWave) {
    const uint16_t* kc = k_cache + (size_t(g) * n_cap + t0) * head_dim + d;
    uint16_t bmn = kc[0], bmx = kc[0];
    float mn = bf16_to_f32(bmn), mx = mn;
    for (int t = t0 + 1; t < t1; ++t) {
      const uint16_t u = kc[size_t(t - t0) * head_dim];
      const float f = bf16_to_f32(u);
      if (f < mn) { mn = f; bmn = u; }
      if (f > mx) { mx = f; bmx = u; }
    }
    uint16_t* sp = summary + ((size_t(g) * (n_cap / 16) + blk) * head_dim + d) * 2;
    sp[0] = bmn;
    sp[1] = bmx;
  }
}

template <int D, bool QP, int NIT>
int launch_score_dqn(const KvSelectParams& p, hipStream_t s) {
  dim3 grid(max(1, ceil_div(p.bud.n_cand, p.score_bpg)), p.n_kv_heads), block(kScoreThreads);
  switch (p.n_heads / p.n_kv_heads) {
    case 1: k_kv_score<D, 1, QP, NIT><<<grid, block, 0, s>>>(p); break;
    case 2: k_kv_score<D, 2, QP, NIT><<<grid, block, 0, s>>>(p); break;
    case 4: k_kv_score<D, 4, QP, NIT><<<grid, block, 0, s>>>(p); break;
    case 8: k_kv_score<D, 8, QP, NIT><<<grid, block, 0, s>>>(p); break;
    default: return set_error(BC_ERR_UNSUPPORTED, "kv score: group %d", p.n_heads / p.n_kv_heads);
  }
  return check_launch("k_kv_score");
}

// 256 blocks per work-group while one round of work-groups covers the
// candidates; beyond that as many as spread them over that round (a
// multiple of one wave load of all 16 waves, at most 1.5 x 256); past that,
// 256 per work-group again in more rounds
template <int D, bool QP>
int launch_score_dq(const KvSelectParams& p_in, hipStream_t s) {
  constexpr int UNIT = (kScoreThreads / kWave) * (kWave / (D / 4));   // blocks per wave load of every wave
  constexpr int NIT1 = kScoreBlocksPerGroup / UNIT;
  KvSelectParams p = p_in;
  const int groups = max(1, kScoreTargetGroups / max(1, p.n_kv_heads));   // per KV head
  const int n = max(1, p.bud.n_cand);
  if (ceil_div(n, kScoreBlocksPerGroup) <= groups) {
    p.score_bpg = kScoreBlocksPerGroup;
    return launch_score_dqn<D, QP, NIT1>(p, s);
  }
  constexpr int NIT2 = NIT1 + NIT1 / 2;   // all issued before q is formed: its registers still fit
  const int bpg = ceil_div(ceil_div(n, groups), UNIT) * UNIT;
  if (bpg <= NIT2 * UNIT) {
    p.score_bpg = bpg;
    return launch_score_dqn<D, QP, NIT2>(p, s);
  }
  p.score_bpg = kScoreBlocksPerGroup;   // more rounds of work-groups
  return launch_score_dqn<D, QP, NIT1>(p, s);
}

}  // namespace

int launch_kv_score(const KvSelectParams& p, hipStream_t s) {
  const bool qp = p.qkv_partial != nullptr;
  if (qp && (p.qkv_splits < 1 || p.qkv_splits > kQkvMaxChunks))
    return set_error(BC_ERR_INVALID, "kv score: %d q/k/v chunks (1..%d)", p.qkv_splits, kQkvMaxChunks);
  if (!qp && (p.bud.n_cand <= 0 || p.bud.k_blk <= 0)) return BC_OK;   // nothing to score
  if (p.head_dim == 128) return qp ? launch_score_dq<128, true>(p, s) : launch_score_dq<128, false>(p, s);
  if (p.head_dim == 64) return qp ? launch_score_dq<64, true>(p, s) : launch_score_dq<64, false>(p, s);
  return set_error(BC_ERR_UNSUPPORTED, "kv score: head_dim %d", p.head_dim);
}

int launch_kv_block_select(const KvSelectParams& p, hipStream_t s) {
  if (p.bud.n_cand > kSelMaxCand) return set_error(BC_ERR_UNSUPPORTED, "kv select: %d candidate blocks", p.bud.n_cand);
  k_kv_block_select<<<dim3(p.n_kv_heads), dim3(kSelThreads), 0, s>>>(p);
  return check_launch("k_kv_block_select");
}

int launch_kv_score_select(const KvSelectParams& p, hipStream_t s) {
  if (p.bud.n_cand > kSelMaxCand) return set_error(BC_ERR_UNSUPPORTED, "kv select: %d candidate blocks", p.bud.n_cand);
  int rc = launch_kv_score(p, s);
  if (rc != BC_OK) return rc;
  return launch_kv_block_select(p, s);
}

}  // namespace bc

using namespace bc;

extern "C" int bc_kv_budget(int n_ctx, const bc_kv_policy* pol, bc_kv_budget_info* out) {
  if (!pol || !out || n_ctx < 0) return set_error(BC_ERR_INVALID, "bc_kv_budget: bad arguments");
  if (pol->block != 16) return set_error(BC_ERR_UNSUPPORTED, "bc_kv_budget: block must be 16");
  if (pol->sinks < 0 || pol->window < 0 || !(pol->r_kv >= 0.0))
    return set_error(BC_ERR_INVALID, "bc_kv_budget: sinks/window/r_kv out of range");
  if (pol->r_kv >= 1.0) {
    *out = bc_kv_budget_info{n_ctx, 0, 0, 0, 0, 0};
    return BC_OK;
  }
  long long T = static_cast<long long>(floor(pol->r_kv * double(n_ctx) + 0.5));
  if (T > n_ctx) T = n_ctx;
  if (T < 0) T = 0;
  const int t = static_cast<int>(T);
  const int sp = pol->sinks < t ? pol->sinks : t;
  const int wp = pol->window < t - sp ? pol->window : t - sp;
  int kb = (t - sp - wp) / 16;
  const int b_lo = (sp + 15) / 16;
  const int b_hi = (n_ctx - wp) / 16;
  const int nc = b_hi > b_lo ? b_hi - b_lo : 0;
  if (kb > nc) kb = nc;
  *out = bc_kv_budget_info{sp + wp + 16 * kb, kb, nc, b_lo, sp, wp};
  return BC_OK;
}

extern "C" size_t bc_kv_score_select_workspace_bytes(int n_ctx, int n_kv_heads, const bc_kv_policy* pol) {
  bc_kv_budget_info b;
  if (n_kv_heads <= 0 || bc_kv_budget(n_ctx, pol, &b) != BC_OK) return 0;
  return align_up(size_t(n_kv_heads) * (b.n_cand > 0 ? b.n_cand : 1) * 4, 256);
}

extern "C" int bc_kv_score_select(const uint16_t* q, const uint16_t* summary, int nb_cap, int n_ctx, int n_heads,
                                  int n_kv_heads, int head_dim, const bc_kv_policy* pol, int32_t* idx_out,
                                  float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !summary || !pol || !idx_out) return set_error(BC_ERR_INVALID, "bc_kv_score_select: NULL pointer");
  if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return set_error(BC_ERR_INVALID, "bc_kv_score_select: heads %d / %d", n_heads, n_kv_heads);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (!valid_group(n_heads / n_kv_heads)) return set_error(BC_ERR_UNSUPPORTED, "group %d", n_heads / n_kv_heads);
  if (n_ctx < 1 || nb_cap * 16 < n_ctx) return set_error(BC_ERR_INVALID, "bc_kv_score_select: n_ctx=%d nb_cap=%d", n_ctx, nb_cap);
  if (pol->r_kv >= 1.0) return set_error(BC_ERR_INVALID, "bc_kv_score_select: r_kv >= 1 needs no selection");
  bc_kv_budget_info b;
  int rc = bc_kv_budget(n_ctx, pol, &b);
  if (rc != BC_OK) return rc;
  float* scores = scores_out;
  if (scores == nullptr) {
    size_t need = bc_kv_score_select_workspace_bytes(n_ctx, n_kv_heads, pol);
    if (!ws || ws_bytes < need) return set_error(BC_ERR_WORKSPACE, "bc_kv_score_select: workspace %zu < %zu", ws_bytes, need);
    scores = static_cast<float*>(ws);
  }
  KvSelectParams p{};
  p.q = q; p.summary = const_cast<uint16_t*>(summary); p.nb_cap = nb_cap; p.n_ctx = n_ctx; p.n_heads = n_heads;
  p.n_kv_heads = n_kv_heads; p.head_dim = head_dim; p.bud = b; p.scores = scores; p.scores_stride = b.n_cand;
  p.idx_out = idx_out;
  return launch_kv_score_select(p, static_cast<hipStream_t>(stream));
}

extern "C" int bc_kv_compact(const uint16_t* k_cache, const uint16_t* v_cache, int n_cap, int n_kv_heads,
                             int head_dim, const int32_t* idx, int t_sel, uint16_t* k_out, uint16_t* v_out,
                             int n_cap_out, void* stream) {
  if (!k_cache || !v_cache || !idx || !k_out || !v_out) return set_error(BC_ERR_INVALID, "bc_kv_compact: NULL pointer");
  if (n_kv_heads <= 0 || n_cap <= 0 || t_sel < 0 || t_sel > n_cap_out)
    return set_error(BC_ERR_INVALID, "bc_kv_compact: n_kv_heads=%d n_cap=%d t_sel=%d n_cap_out=%d", n_kv_heads, n_cap,
                     t_sel, n_cap_out);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  const long long pieces = (long long)t_sel * (head_dim / 8);
  if (pieces == 0) return BC_OK;
  k_kv_compact<<<dim3(unsigned((pieces + 255) / 256), n_kv_heads), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      k_cache, v_cache, n_cap, head_dim, idx, t_sel, k_out, v_out, n_cap_out);
  return check_launch("k_kv_compact");
}

extern "C" int bc_build_kv_summary(const uint16_t* k_cache, int n_kv_heads, int n_cap, int head_dim, int n_ctx,
                                   uint16_t* summary, void* stream) {
  if (!k_cache || !summary) return set_error(BC_ERR_INVALID, "bc_build_kv_summary: NULL pointer");
  if (n_kv_heads <= 0 || n_cap <= 0 || n_cap % 16 != 0 || n_ctx < 0 || n_ctx > n_cap)
    return set_error(BC_ERR_INVALID, "bc_build_kv_summary: n_kv_heads=%d n_cap=%d n_ctx=%d", n_kv_heads, n_cap, n_ctx);
  if (!valid_head_dim(head_dim)) return set_error(BC_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  const int nb = (n_ctx + 15) / 16;
  if (nb == 0) return BC_OK;
  k_build_summary<<<dim3(ceil_div(nb, 4), n_kv_heads), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      k_cache, n_cap, head_dim, n_ctx, summary);
  return check_launch("k_build_summary");
}
