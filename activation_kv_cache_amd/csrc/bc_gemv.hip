// bc_gemv.hip -- activation-sparse projection GEMV for gfx950.
//
// y[o] = sum_{j<k} W^T[idx_j][o] * x[idx_j]  (README "What it does in one
// picture": each token's activations select the weight columns read).
//
// W^T is [d_in][d_out] bf16: the weights of one input channel are one row,
// stored tile-major (128-column tiles, each tile's rows contiguous).  A
// work-group owns one 128-column tile of y and one chunk of list positions.
// Its 1024 lanes form 64 row slots of 16 lanes; a slot reads a row's 256 B
// with one 16-byte load per lane.  Each slot keeps a ring of 2 rows in
// flight (32 KB per work-group), issued as non-temporal loads: the weights
// are read once per step and should not evict the small vectors the kernels
// share.
// Sixteen waves (four per SIMD) also split the prologue's selection work
// finely and hide its LDS and memory latency.
//
// The prologue forms the input.  IN_NORM computes x = RMSNorm(h) * gain
// (IN_NORM_SUM first forms h from the previous GEMV's chunk partials and a
// residual) and IN_SEL takes x as given; with k < d_in both then select the
// exact top-k of |x| (block_topk_2pass) in every work-group, so no separate
// selection kernel or single-work-group stage sits between two GEMVs.
// IN_ATTN (dense) forms the chunk's channels of x from attention split
// partials, IN_LIST takes x and an optional channel list as given.  The
// first ring of weight loads goes out right after the prologue's own loads,
// before its arithmetic (for a selection, once the list is known).
//
// Several chunks write fp32 partials ([chunk][d_out]); a finish kernel adds
// them in chunk order (deterministic) and applies the epilogue: bf16 store,
// residual add, rotary + KV append + block summary, SwiGLU, or logits +
// argmax.  With one chunk the main kernel applies the bf16, SwiGLU or argmax
// epilogue itself.  No work-group waits for another: cross-XCD fences cost
// far more on this chip than a kernel boundary.
#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include "bc_clock.hpp"
#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

constexpr int kSlots = kGemvThreads / 16;   // 64 row slots of 16 lanes
// rows in flight per slot (32 KB per work-group): 2 measured 2-4% faster
// than 4, and 6 or 8 slower still
template <int OUT>
constexpr int ring_depth() { return 2; }
constexpr int kNW = kGemvThreads / kWave;   // 16 waves
constexpr int kTopkShift = 3;               // first selection pass: 4096 bins
// IN_ATTN: one thread per channel (rows_per_split <= kGemvThreads), so a
// chunk spans at most kGemvThreads / 64 + 1 heads (head_dim >= 64)
constexpr int kFoldMaxHeads = kGemvThreads / 64 + 1;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct GemvSmem {
  struct {
    int32_t ch[kGemvMaxRows];   // channel of each list position of the chunk
    float xv[kGemvMaxRows];     // its input value
  } list;
  float red[kNW][kGemvTile];    // per-wave column sums (after the row loop)
  union {
    Topk2Smem<kGemvThreads, kTopkShift> tk;
    struct {
      alignas(16) float w[kFoldMaxHeads][kAttnFoldMaxSplits];   // combine weights w_s per head of the chunk
      float den[kFoldMaxHeads];
    } fold;
  };
  float part[kNW];
  float amax_v[kNW];
  int32_t amax_i[kNW];
};

// Input values per thread in the fused prologue: a multiple of 4 (8-byte
// loads), thread t owning channels [t*P, t*P + P).
__host__ __device__ inline int fused_per_thread(int d_in) {
  return ((d_in + kGemvThreads - 1) / kGemvThreads + 3) & ~3;
}

__device__ __forceinline__ u32x4 load_row_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_elt(const uint32_t* packed, int e) {
  return (e & 1) ? bf16_hi(packed[e >> 1]) : bf16_lo(packed[e >> 1]);
}

template <int PMAX>
__device__ __forceinline__ void load_vec(const uint16_t* src, int c0, int P, int d_in, uint32_t (&dst)[PMAX / 2]) {
#pragma unroll
  for (int q = 0; q < PMAX / 4; ++q) {
    uint2 v = make_uint2(0u, 0u);
    if (4 * q < P && c0 + 4 * q < d_in) v = *reinterpret_cast<const uint2*>(src + c0 + 4 * q);
    dst[2 * q] = v.x;
    dst[2 * q + 1] = v.y;
  }
}

// h = bf16(sum of the chunk partials in chunk order + resid) for the thread's
// channels [c0, c0 + P): the arithmetic of k_finish_resid.  sum_load issues
// the loads of the first 8 chunks and of resid, sum_finish adds them (and
// any further chunks).  Channels past d_in give 0.
template <int PMAX>
struct SumIn {
  float4 a[PMAX / 4][8];
  uint2 rv[PMAX / 4];
};

template <int PMAX>
__device__ __forceinline__ void sum_load(const float* partial, int n_splits, const uint16_t* resid, int c0, int P,
                                         int d_in, SumIn<PMAX>& in) {
#pragma unroll
  for (int q = 0; q < PMAX / 4; ++q) {
    const bool ok = 4 * q < P && c0 + 4 * q < d_in;
    const int c = ok ? c0 + 4 * q : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      in.a[q][u] = *reinterpret_cast<const float4*>(partial + size_t(min(u, n_splits - 1)) * d_in + c);
    in.rv[q] = *reinterpret_cast<const uint2*>(resid + c);
  }
}

template <int PMAX>
__device__ __forceinline__ void sum_finish(const float* partial, int n_splits, int c0, int P, int d_in,
                                           const SumIn<PMAX>& in, uint32_t (&dst)[PMAX / 2]) {
#pragma unroll
  for (int q = 0; q < PMAX / 4; ++q) {
    const bool ok = 4 * q < P && c0 + 4 * q < d_in;
    const int c = ok ? c0 + 4 * q : 0;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < n_splits) {
        v.x += in.a[q][u].x; v.y += in.a[q][u].y; v.z += in.a[q][u].z; v.w += in.a[q][u].w;
      }
    }
    for (int sp = 8; sp < n_splits; ++sp) {
      const float4 b = *reinterpret_cast<const float4*>(partial + size_t(sp) * d_in + c);
      v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
    }
    const uint2 rv = in.rv[q];
    v.x += bf16_lo(rv.x); v.y += bf16_hi(rv.x); v.z += bf16_lo(rv.y); v.w += bf16_hi(rv.y);
    dst[2 * q] = ok ? (f32_to_bf16(v.x) | (uint32_t(f32_to_bf16(v.y)) << 16)) : 0u;
    dst[2 * q + 1] = ok ? (f32_to_bf16(v.z) | (uint32_t(f32_to_bf16(v.w)) << 16)) : 0u;
  }
}

template <int IN, int OUT, int PMAX>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(const GemvParams p) {
  constexpr int kRing = ring_depth<OUT>();
  __shared__ GemvSmem sm;
  // phase ends (a build with phase clocks only): [3] inputs arrived, [4]
  // input formed (after its barrier), [5..9] the selection's barriers, [10]
  // selection emitted, [11] prologue done, [12] row loop done
  PhaseClock clk;
  clk.begin();
  const int tile = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = tid & 15, slot = tid >> 4;
  const int r0 = split * p.rows_per_split;
  const int r1 = min(p.k, r0 + p.rows_per_split);
  const int n = r1 - r0;   // >= 1 (plan_gemv)
  const bool dense = (IN == IN_LIST) ? p.idx == nullptr : p.k == p.d_in;
  const bool lead = blockIdx.x == 0 && blockIdx.y == 0;
  const int tile_w = min(kGemvTile, p.d_out - tile * kGemvTile);
  const bool col_ok = l16 * 8 < tile_w;
  // lanes past a narrow last tile read the tile's first columns (discarded)
  const uint16_t* base;
  size_t stride;
  if (p.tiled) {
    base = p.wt + size_t(tile) * kGemvTile * p.d_in + (col_ok ? l16 * 8 : 0);
    stride = size_t(tile_w);
  } else {
    base = p.wt + size_t(tile) * kGemvTile + (col_ok ? l16 * 8 : 0);
    stride = size_t(p.d_out);
  }
  // list position j -> its row; positions past the chunk re-read its last
  // row, so every slot issues the same sequence of loads.  Row
  // ids are clamped to the matrix, so a bad id cannot read outside it.
  const unsigned last_row = unsigned(p.d_in - 1);
  auto row_ptr = [&](int j) -> const uint16_t* {
    const int jj = min(j, n - 1);
    const unsigned ch = dense ? unsigned(r0 + jj) : min(unsigned(sm.list.ch[jj]), last_row);
    return base + size_t(ch) * stride;
  };
  // A dense chunk's first ring goes out right after the prologue's own
  // loads: a wave's loads complete in issue order, so the inputs the
  // prologue waits for are not queued behind its share of the weights, and
  // the weights stream while the prologue computes.
  u32x4 ring[kRing];
  auto issue_ring = [&]() {
#pragma unroll
    for (int u = 0; u < kRing; ++u) ring[u] = load_row_nt(row_ptr(slot + kSlots * u));
  };

  // ------------------------------------------------------------ prologue
  // Instantiated for dense and for selected chunks separately, so that the
  // compiler counts the outstanding loads of each path exactly (a merged
  // path would wait for the first ring before using the prologue's loads).
  auto prologue = [&](auto dense_tag) {
    constexpr bool DENSE = decltype(dense_tag)::value;
    if constexpr (IN == IN_LIST) {
      if (DENSE) {
        constexpr int Q = kGemvMaxRows / kGemvThreads;
        float xq[Q];
        // clamped, unconditional loads: no branch separates a load from its use
#pragma unroll
        for (int q = 0; q < Q; ++q) xq[q] = bf16_to_f32(p.x[r0 + min(tid + q * kGemvThreads, n - 1)]);
        issue_ring();
        clk.stamp_after(3, xq[Q - 1]);
#pragma unroll
        for (int q = 0; q < Q; ++q)
          if (tid + q * kGemvThreads < n) sm.list.xv[tid + q * kGemvThreads] = xq[q];
      } else {
        // the list entries (the thread's, then its slot's first ring rows),
        // then x at the thread's entries, then the first ring straight from
        // the entries in registers: the weights stream while the list is
        // staged in LDS
        constexpr int Q = kGemvMaxRows / kGemvThreads;
        unsigned chq[Q], chr[kRing];
        float xq[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) chq[q] = unsigned(p.idx[r0 + min(tid + q * kGemvThreads, n - 1)]);
#pragma unroll
        for (int u = 0; u < kRing; ++u)
          chr[u] = min(unsigned(p.idx[r0 + min(slot + kSlots * u, n - 1)]), last_row);
#pragma unroll
        for (int q = 0; q < Q; ++q) xq[q] = bf16_to_f32(p.x[min(chq[q], last_row)]);
#pragma unroll
        for (int u = 0; u < kRing; ++u) ring[u] = load_row_nt(base + size_t(chr[u]) * stride);
        clk.stamp_after(3, xq[Q - 1]);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const int j = tid + q * kGemvThreads;
          if (j < n) {
            sm.list.ch[j] = int(chq[q]);
            sm.list.xv[j] = xq[q];
          }
        }
      }
    } else if constexpr (IN == IN_ATTN) {
      // x of channels [r0, r1) from the attention split partials, in the
      // combine order of k_attn_reduce: thread j owns channel r0 + j and loads
      // its S values of o first; one wave per head of the chunk forms w_s and
      // den (lane s holds split s)
      const int D = p.a_hd, S = p.a_splits;
      const int h0 = r0 / D, nh = (r1 - 1) / D - h0 + 1;
      const int c = r0 + min(tid, n - 1);
      const int hh = c / D - h0;
      // wave w's first head: its m and l go out first, then o, then the ring
      float ms0 = -INFINITY, lv0 = 0.f;
      if (w < nh && lane < S) {
        ms0 = p.am[size_t(h0 + w) * S + lane];
        lv0 = p.al[size_t(h0 + w) * S + lane];
      }
      const float* osrc = p.ao + size_t(c / D) * S * D + (c % D);
      float ov[kAttnFoldMaxSplits];
#pragma unroll
      for (int sp = 0; sp < kAttnFoldMaxSplits; ++sp) ov[sp] = osrc[size_t(min(sp, S - 1)) * D];
      issue_ring();
      clk.stamp_after(3, ov[kAttnFoldMaxSplits - 1]);
      auto head_weights = [&](int hw, float ms, float lv) {
        float M = ms;
        M = wave_max_f32(M);
        const float wt = combine_weight(ms, M);
        const float den = combine_wave_sum(lane < S ? fmaf(wt, lv, 0.f) : 0.f);
        if (lane < S) sm.fold.w[hw][lane] = wt;
        if (lane == 0) sm.fold.den[hw] = 0.f + den;
      };
      // the first head from the values loaded above: no load of the same
      // address sits in a loop behind the weight rows, where waiting for it
      // would mean waiting for them too
      if (w < nh) head_weights(w, ms0, lv0);
      // more heads than waves (head_dim 64, 17 heads): loaded here
      for (int hw = w + kNW; hw < nh; hw += kNW) {
        const size_t hb = size_t(h0 + hw) * S;
        head_weights(hw, lane < S ? p.am[hb + lane] : -INFINITY, lane < S ? p.al[hb + lane] : 0.f);
      }
      __syncthreads();
      clk.stamp(4);
      if (tid < n) {
        const int G = kCombineThreads / D, per = (S + G - 1) / G;
        // the head's weights in registers first (16-byte LDS reads, one
        // wait), so the sums below do not wait on LDS split by split
        float wr[kAttnFoldMaxSplits];
        const float4* wv4 = reinterpret_cast<const float4*>(sm.fold.w[hh]);
#pragma unroll
        for (int q = 0; q < kAttnFoldMaxSplits / 4; ++q) {
          const float4 v4 = wv4[q];
          wr[4 * q] = v4.x;
          wr[4 * q + 1] = v4.y;
          wr[4 * q + 2] = v4.z;
          wr[4 * q + 3] = v4.w;
        }
        float t = 0.f;
        if (S == kAttnFoldMaxSplits && (G == 2 || G == 4)) {
          // every split present (the usual case): each group's splits are
          // known, so the sums take no selects; the same fmaf chains and the
          // same group order as below
          static_assert(kAttnFoldMaxSplits % 4 == 0, "groups of whole splits");
          float nm[4] = {0.f, 0.f, 0.f, 0.f};
          if (G == 2) {
#pragma unroll
            for (int i = 0; i < kAttnFoldMaxSplits / 2; ++i) {
              nm[0] = fmaf(ov[i], wr[i], nm[0]);
              nm[1] = fmaf(ov[kAttnFoldMaxSplits / 2 + i], wr[kAttnFoldMaxSplits / 2 + i], nm[1]);
            }
            t += nm[0];
            t += nm[1];
          } else {
#pragma unroll
            for (int i = 0; i < kAttnFoldMaxSplits / 4; ++i)
#pragma unroll
              for (int g = 0; g < 4; ++g)
                nm[g] = fmaf(ov[g * (kAttnFoldMaxSplits / 4) + i], wr[g * (kAttnFoldMaxSplits / 4) + i], nm[g]);
#pragma unroll
            for (int g = 0; g < 4; ++g) t += nm[g];
          }
        } else {
          for (int g = 0; g < G; ++g) {
            const int s0 = min(S, g * per), s1 = min(S, s0 + per);
            // combine_group over registers: splits outside [s0, s1) leave the
            // sum as it is (their weights are not set; the select drops them)
            float num = 0.f;
#pragma unroll
            for (int sp = 0; sp < kAttnFoldMaxSplits; ++sp) {
              const float nx = fmaf(ov[sp], wr[sp], num);
              num = (sp >= s0 && sp < s1) ? nx : num;
            }
            t += num;
          }
        }
        const float den = sm.fold.den[hh];
        const uint32_t xb = f32_to_bf16(den > 0.f ? t / den : 0.f);
        sm.list.xv[tid] = __uint_as_float(xb << 16);
        if (tile == 0 && p.x_out) p.x_out[c] = uint16_t(xb);
      }
    } else {
      const int P = fused_per_thread(p.d_in);
      const int c0 = tid * P;
      uint32_t xb[PMAX / 2];
      if constexpr (IN == IN_NORM || IN == IN_NORM_SUM) {
        uint32_t gb[PMAX / 2];
        [[maybe_unused]] SumIn<(IN == IN_NORM_SUM ? PMAX : 4)> sin;
        if constexpr (IN == IN_NORM_SUM) sum_load<PMAX>(p.sum_partial, p.sum_splits, p.h, c0, P, p.d_in, sin);
        if constexpr (IN == IN_NORM) load_vec<PMAX>(p.h, c0, P, p.d_in, xb);
        load_vec<PMAX>(p.gain, c0, P, p.d_in, gb);
        if (DENSE) issue_ring();
        if (!DENSE) topk2_clear(sm.tk);   // while the loads are in flight; the barrier below covers it
        clk.stamp_after(3, __uint_as_float(gb[PMAX / 2 - 1]));
        if constexpr (IN == IN_NORM_SUM) {
          sum_finish<PMAX>(p.sum_partial, p.sum_splits, c0, P, p.d_in, sin, xb);
          if (lead && p.h_out) {
#pragma unroll
            for (int q = 0; q < PMAX / 4; ++q)
              if (4 * q < P && c0 + 4 * q < p.d_in)
                *reinterpret_cast<uint2*>(p.h_out + c0 + 4 * q) = make_uint2(xb[2 * q], xb[2 * q + 1]);
          }
        }
        // sum of squares in a fixed order: the thread's channels in order, the
        // wave's fixed tree, then the waves in order (all work-groups agree)
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < PMAX; ++e) {
          const float v = bf16_elt(xb, e);
          ss += v * v;   // channels past d_in were loaded as 0
        }
        ss = wave_sum_f32(ss);
        if (lane == 0) sm.part[w] = ss;
        __syncthreads();
        clk.stamp(4);
        float tot = 0.f;
#pragma unroll
        for (int ww = 0; ww < kNW; ++ww) tot += sm.part[ww];
        const float inv = 1.0f / sqrtf(tot / float(p.d_in) + p.eps);
#pragma unroll
        for (int q = 0; q < PMAX / 2; ++q) {
          const uint32_t a = f32_to_bf16(bf16_lo(xb[q]) * inv * bf16_lo(gb[q]));
          const uint32_t b = f32_to_bf16(bf16_hi(xb[q]) * inv * bf16_hi(gb[q]));
          xb[q] = a | (b << 16);
        }
      } else {
        load_vec<PMAX>(p.x, c0, P, p.d_in, xb);
        if (DENSE) issue_ring();
        clk.stamp_after(3, __uint_as_float(xb[PMAX / 2 - 1]));
        if (!DENSE) {
          topk2_clear(sm.tk);
          __syncthreads();
          clk.stamp(4);
        }
      }
      if (lead && p.x_out) {
#pragma unroll
        for (int q = 0; q < PMAX / 4; ++q)
          if (4 * q < P && c0 + 4 * q < p.d_in)
            *reinterpret_cast<uint2*>(p.x_out + c0 + 4 * q) = make_uint2(xb[2 * q], xb[2 * q + 1]);
      }
      if (DENSE) {
#pragma unroll
        for (int e = 0; e < PMAX; ++e) {
          const int c = c0 + e;
          if (e < P && c >= r0 && c < r1) sm.list.xv[c - r0] = bf16_elt(xb, e);
        }
      } else {
        uint32_t key[PMAX];
#pragma unroll
        for (int e = 0; e < PMAX; ++e) key[e] = ((xb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) & 0x7FFFu;
        int32_t* idx_out = p.idx_out;
        auto emit = [&](int rel, int e) {
          sm.list.ch[rel] = c0 + e;
          sm.list.xv[rel] = bf16_elt(xb, e);
        };
        auto out = [&](int pos, int e) { idx_out[pos] = c0 + e; };
        auto stamp = [&](int phase) { clk.stamp(5 + phase); };
        block_topk_2pass<kGemvThreads, kTopkShift, PMAX>(key, P, p.d_in, p.k, r0, r1, emit, sm.tk,
                                                         lead && idx_out != nullptr, out, stamp);
      }
    }
  };
  if (dense)
    prologue(std::true_type{});
  else
    prologue(std::false_type{});
  __syncthreads();
  if (IN != IN_LIST && !dense) issue_ring();
  clk.stamp(11);

  // ------------------------------------------------------------- row loop
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  auto consume = [&](int j, const u32x4& wv) {
    const float x = j < n ? sm.list.xv[j] : 0.f;
    acc[0] += bf16_lo(wv.x) * x;
    acc[1] += bf16_hi(wv.x) * x;
    acc[2] += bf16_lo(wv.y) * x;
    acc[3] += bf16_hi(wv.y) * x;
    acc[4] += bf16_lo(wv.z) * x;
    acc[5] += bf16_hi(wv.z) * x;
    acc[6] += bf16_lo(wv.w) * x;
    acc[7] += bf16_hi(wv.w) * x;
  };
  // Ring groups of kRing steps; every group but the last refills its slot
  // with the row kRing steps ahead.  The last group only consumes: its
  // refills would all lie past the chunk, and waiting for them would add a
  // memory round trip to the end of every work-group.
  const int nsteps = (n + kSlots - 1) / kSlots;
  int st = 0;
  for (; st + kRing < nsteps; st += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int j = slot + kSlots * (st + u);
      consume(j, ring[u]);
      ring[u] = load_row_nt(row_ptr(j + kSlots * kRing));
    }
  }
#pragma unroll
  for (int u = 0; u < kRing; ++u) consume(slot + kSlots * (st + u), ring[u]);

  clk.stamp_after(12, acc[7]);

  // ------------------------------------------------------------- epilogue
  // The four slots of a wave (its 16-lane rows) hold the same 8 columns:
  // they are summed across rows in registers (lane ^ 32, then lane ^ 16),
  // the waves' sums through LDS in wave order.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    acc[c] += lane_xor<32>(acc[c]);
    acc[c] += lane_xor<16>(acc[c]);
  }
  if (lane < 16) {
    float4* rw = reinterpret_cast<float4*>(&sm.red[w][l16 * 8]);
    rw[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    rw[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  auto col_sum = [&](int c) {
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) v += sm.red[ww][c];
    return v;
  };
  if constexpr (OUT == OUT_PARTIAL) {
    if (tid < tile_w) p.partial[size_t(split) * p.d_out + tile * kGemvTile + tid] = col_sum(tid);
  } else if constexpr (OUT == OUT_BF16) {
    if (tid < tile_w) p.y[tile * kGemvTile + tid] = f32_to_bf16(col_sum(tid));
  } else if constexpr (OUT == OUT_SWIGLU) {
    // tile t: gate columns [0, wu) and up columns [wu, 2 wu) of hidden units
    // [64t, 64t + wu)
    const int wu = tile_w / 2;
    if (tid < wu) {
      const float g = col_sum(tid), u = col_sum(wu + tid);
      p.y[tile * (kGemvTile / 2) + tid] = f32_to_bf16(g / (1.0f + expf(-g)) * u);
    }
  } else {
    float best = -INFINITY;
    int besti = 0x7FFFFFFF;
    if (tid < tile_w) {
      const int c = tile * kGemvTile + tid;
      best = col_sum(tid);
      besti = c;
      p.yf[c] = best;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(best, off, kWave);
      const int oi = __shfl_xor(besti, off, kWave);
      if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
    }
    if (lane == 0) { sm.amax_v[w] = best; sm.amax_i[w] = besti; }
    __syncthreads();
    if (tid == 0) {
      for (int ww = 1; ww < kNW; ++ww) {
        const float ov = sm.amax_v[ww];
        const int oi = sm.amax_i[ww];
        if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
      }
      p.tile_max[tile] = best;
      p.tile_arg[tile] = besti;
    }
  }
  clk.end(p.clk, size_t(split) * gridDim.x + tile);
}

// ------------------------------------------------------------------ finish
__global__ __launch_bounds__(256) void k_finish_bf16(const FinishParams p) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < p.d_out) p.y[c] = f32_to_bf16(chunk_sum(p.partial, p.n_splits, p.d_out, c));
}

// y = bf16(sum of chunks + resid), one column per thread.
__global__ __launch_bounds__(128) void k_finish_resid(const FinishParams p) {
  const int c = blockIdx.x * 128 + threadIdx.x;
  if (c >= p.d_out) return;
  float v = chunk_sum(p.partial, p.n_splits, p.d_out, c);
  if (p.resid) v += bf16_to_f32(p.resid[c]);
  p.y[c] = f32_to_bf16(v);
}

// SwiGLU over the chunk sums of the packed gate | up tiles: tile t holds gate
// columns [128t, 128t + w) and up columns [128t + w, 128t + 2w) of hidden
// units [64t, 64t + w), w = min(64, d_ff - 64t).  One unit per thread.
__global__ __launch_bounds__(256) void k_finish_swiglu(const FinishParams p) {
  const int half = kGemvTile / 2;
  const int u = blockIdx.x * 256 + threadIdx.x;
  if (u >= p.d_ff) return;
  const int t = u / half, off = u % half;
  const int w = min(half, p.d_ff - t * half);
  const float g = chunk_sum(p.partial, p.n_splits, p.d_out, t * kGemvTile + off);
  const float v = chunk_sum(p.partial, p.n_splits, p.d_out, t * kGemvTile + w + off);
  p.y[u] = f32_to_bf16(g / (1.0f + expf(-g)) * v);
}

// Logits from chunk sums, and the argmax of each block of 256 columns.
__global__ __launch_bounds__(256) void k_finish_argmax(const FinishParams p) {
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  const int c = blockIdx.x * 256 + threadIdx.x;
  float best = -INFINITY;
  int besti = 0x7FFFFFFF;
  if (c < p.d_out) {
    best = chunk_sum(p.partial, p.n_splits, p.d_out, c);
    besti = c;
    p.yf[c] = best;
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
    for (int ww = 1; ww < 4; ++ww)
      if (sv[ww] > best || (sv[ww] == best && si[ww] < besti)) { best = sv[ww]; besti = si[ww]; }
    p.tile_max[blockIdx.x] = best;
    p.tile_arg[blockIdx.x] = besti;
  }
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
      const float cs = p.rope.c[i], sn = p.rope.s[i];
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


constexpr int kOneGroup = 1024;

// bc_select_channels: one 1024-lane work-group.  Up to 16384 channels the
// keys sit in registers (16 per thread at most) and block_topk_2pass ranks
// them -- the selection every GEMV work-group runs in its prologue; the
// ascending list is staged in LDS and stored with coalesced writes.  Larger
// inputs take the 4-bit radix select over keys read from memory.
template <int PMAX>
__global__ __launch_bounds__(kOneGroup) void k_select_reg(const uint16_t* x, int n, int k, int32_t* idx_out,
                                                          int x_stride) {
  __shared__ Topk2Smem<kOneGroup, kTopkShift> tk;
  x += size_t(blockIdx.x) * x_stride;       // one work-group per sequence of a batch
  idx_out += size_t(blockIdx.x) * k;
  __shared__ int32_t list[kOneGroup * PMAX];
  const int P = ((n + kOneGroup - 1) / kOneGroup + 3) & ~3;
  const int c0 = int(threadIdx.x) * P;
  topk2_clear<kOneGroup>(tk);
  uint32_t key[PMAX];
  if ((n & 3) == 0 && (reinterpret_cast<uintptr_t>(x) & 7) == 0) {
    // 8-byte loads of 4 channels (n a multiple of 4: a group is all in or out)
#pragma unroll
    for (int q = 0; q < PMAX / 4; ++q) {
      uint2 v = make_uint2(0u, 0u);
      if (4 * q < P && c0 + 4 * q < n) v = *reinterpret_cast<const uint2*>(x + c0 + 4 * q);
      key[4 * q] = v.x & 0x7FFFu;
      key[4 * q + 1] = (v.x >> 16) & 0x7FFFu;
      key[4 * q + 2] = v.y & 0x7FFFu;
      key[4 * q + 3] = (v.y >> 16) & 0x7FFFu;
    }
  } else {
#pragma unroll
    for (int e = 0; e < PMAX; ++e) {
      const int c = c0 + e;
      key[e] = (e < P && c < n) ? (uint32_t(x[c]) & 0x7FFFu) : 0u;
    }
  }
  __syncthreads();
  auto emit = [&](int pos, int e) { list[pos] = c0 + e; };
  block_topk_2pass<kOneGroup, kTopkShift, PMAX>(key, P, n, k, 0, k, emit, tk);
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += kOneGroup) idx_out[i] = list[i];
}

__global__ __launch_bounds__(kOneGroup) void k_select(const uint16_t* x, int n, int k, int32_t* idx_out,
                                                      int x_stride) {
  __shared__ TopkSmem<kOneGroup, uint16_t> sm;
  x += size_t(blockIdx.x) * x_stride;
  idx_out += size_t(blockIdx.x) * k;
  auto key = [x](int i) -> uint32_t { return uint32_t(x[i]) & 0x7FFFu; };
  auto emit = [idx_out](int r, int i) { idx_out[r] = i; };
  block_topk<kOneGroup, 15, uint16_t>(n, k, key, emit, sm);
}


}  // namespace

static int gemv_target_groups() {
  // tuning override for sweeps; the default is one work-group per CU
  static const int v = [] {
    const char* e = getenv("BC_GEMV_GROUPS");
    const int x = e ? atoi(e) : 0;
    return x > 0 ? x : 256;
  }();
  return v;
}

GemvPlan plan_gemv(int d_out, int k, bool single, int max_splits) {
  GemvPlan pl;
  pl.n_tiles = ceil_div(d_out, kGemvTile);
  if (k < 1) k = 1;
  int splits;
  if (single && k <= kGemvMaxRows) {
    splits = 1;
  } else {
    const int target = gemv_target_groups();
    splits = (target + pl.n_tiles / 2) / pl.n_tiles;
    splits = min(splits, k / 64);   // at least 64 rows per chunk
    if (max_splits > 0) splits = min(splits, max_splits);
    splits = max(splits, 1);
    splits = max(splits, ceil_div(k, kGemvMaxRows));
  }
  int rps = ceil_div(k, splits);
  rps = (rps + 15) / 16 * 16;
  pl.rows_per_split = min(rps, kGemvMaxRows);
  pl.n_splits = ceil_div(k, pl.rows_per_split);
  pl.partial_bytes = align_up(size_t(pl.n_splits) * d_out * 4, 256);
  return pl;
}

bool gemv_fused_input_ok(int d_in) { return d_in >= 1 && d_in % 4 == 0 && d_in <= kGemvFusedMaxIn; }

bool gemv_attn_fold_ok(int d_in, int d_out, int head_dim, int attn_splits) {
  if ((head_dim != 64 && head_dim != 128) || d_in < head_dim || d_in % head_dim != 0) return false;
  if (attn_splits < 1 || attn_splits > kAttnFoldMaxSplits) return false;
  return plan_gemv(d_out, d_in).rows_per_split <= kGemvThreads;
}
bool gemv_sum_input_ok(int d_in) { return gemv_fused_input_ok(d_in) && fused_per_thread(d_in) <= 4; }

namespace {
template <int IN, int PMAX>
int launch_gemv_out(int out, const GemvParams& p, dim3 grid, hipStream_t s) {
  const dim3 block(kGemvThreads);
  switch (out) {
    case OUT_PARTIAL: k_gemv<IN, OUT_PARTIAL, PMAX><<<grid, block, 0, s>>>(p); break;
    case OUT_BF16: k_gemv<IN, OUT_BF16, PMAX><<<grid, block, 0, s>>>(p); break;
    case OUT_SWIGLU: k_gemv<IN, OUT_SWIGLU, PMAX><<<grid, block, 0, s>>>(p); break;
    case OUT_ARGMAX: k_gemv<IN, OUT_ARGMAX, PMAX><<<grid, block, 0, s>>>(p); break;
    default: return set_error(BC_ERR_INVALID, "unknown GEMV output %d", out);
  }
  return check_launch("k_gemv");
}
}  // namespace

int launch_gemv(int in, int out, const GemvParams& p_in, hipStream_t s) {
  GemvParams p = p_in;
  p.clk = clock_take(size_t(p.n_tiles) * p.n_splits, CLOCK_GEMV, in | (out << 8), p.d_in, p.d_out, p.k);
  if (p.n_splits < 1 || p.n_tiles < 1 || p.rows_per_split < 1 || p.rows_per_split > kGemvMaxRows ||
      size_t(p.n_splits - 1) * p.rows_per_split >= size_t(p.k) || size_t(p.n_splits) * p.rows_per_split < size_t(p.k))
    return set_error(BC_ERR_INVALID, "GEMV plan does not cover k=%d", p.k);
  if (out != OUT_PARTIAL && p.n_splits != 1) return set_error(BC_ERR_INVALID, "GEMV epilogue needs one chunk");
  if (out == OUT_SWIGLU && ceil_div(p.d_out, kGemvTile) != p.n_tiles)
    return set_error(BC_ERR_INVALID, "SwiGLU epilogue: tile count");
  const dim3 grid(p.n_tiles, p.n_splits);
  if (in == IN_LIST) return launch_gemv_out<IN_LIST, 4>(out, p, grid, s);
  if (in == IN_ATTN) {
    if (p.k != p.d_in || p.idx || !p.am || !p.al || !p.ao || (p.a_hd != 64 && p.a_hd != 128) ||
        p.d_in % p.a_hd != 0 || p.a_splits < 1 || p.a_splits > kAttnFoldMaxSplits ||
        p.rows_per_split > kGemvThreads || (out != OUT_PARTIAL && out != OUT_BF16))
      return set_error(BC_ERR_INVALID, "IN_ATTN: d_in=%d k=%d head_dim=%d splits=%d", p.d_in, p.k, p.a_hd,
                       p.a_splits);
    if (out == OUT_PARTIAL)
      k_gemv<IN_ATTN, OUT_PARTIAL, 4><<<grid, dim3(kGemvThreads), 0, s>>>(p);
    else
      k_gemv<IN_ATTN, OUT_BF16, 4><<<grid, dim3(kGemvThreads), 0, s>>>(p);
    return check_launch("k_gemv");
  }
  if (in != IN_NORM && in != IN_SEL && in != IN_NORM_SUM) return set_error(BC_ERR_INVALID, "unknown GEMV input %d", in);
  if (!gemv_fused_input_ok(p.d_in)) return set_error(BC_ERR_UNSUPPORTED, "fused GEMV input d_in=%d", p.d_in);
  static_assert(kGemvFusedMaxIn <= kGemvThreads * 16, "fused inputs fit 16 per thread");
  const bool big = fused_per_thread(p.d_in) > 4;
  if (in == IN_NORM_SUM) {
    if (big || !p.sum_partial || !p.h || p.sum_splits < 1)
      return set_error(BC_ERR_INVALID, "IN_NORM_SUM: d_in=%d, %d chunks", p.d_in, p.sum_splits);
    return launch_gemv_out<IN_NORM_SUM, 4>(out, p, grid, s);
  }
  if (in == IN_NORM)
    return big ? launch_gemv_out<IN_NORM, 16>(out, p, grid, s) : launch_gemv_out<IN_NORM, 4>(out, p, grid, s);
  return big ? launch_gemv_out<IN_SEL, 16>(out, p, grid, s) : launch_gemv_out<IN_SEL, 4>(out, p, grid, s);
}

int finish_argmax_groups(int d_out) { return ceil_div(d_out, 256); }

int launch_finish(int kind, const FinishParams& p, hipStream_t s) {
  switch (kind) {
    case FIN_BF16: k_finish_bf16<<<ceil_div(p.d_out, 256), 256, 0, s>>>(p); break;
    case FIN_QKV: k_finish_qkv<<<p.n_heads + 2 * p.n_kv_heads, 64, 0, s>>>(p); break;
    case FIN_RESID: k_finish_resid<<<ceil_div(p.d_out, 128), 128, 0, s>>>(p); break;
    case FIN_SWIGLU: k_finish_swiglu<<<ceil_div(p.d_ff, 256), 256, 0, s>>>(p); break;
    case FIN_ARGMAX: k_finish_argmax<<<finish_argmax_groups(p.d_out), 256, 0, s>>>(p); break;
    default: return set_error(BC_ERR_INVALID, "unknown finish kind %d", kind);
  }
  return check_launch("k_finish");
}

int launch_argmax_finish(const float* tile_max, const int32_t* tile_arg, int n_tiles, int32_t* token, hipStream_t s) {
  k_argmax_finish<<<1, 256, 0, s>>>(tile_max, tile_arg, n_tiles, token);
  return check_launch("k_argmax_finish");
}

int launch_select_batch(const uint16_t* x, int n, int k, int32_t* idx_out, int batch, int x_stride, hipStream_t s) {
  const dim3 grid{unsigned(batch)};
  if (n <= kOneGroup * 4)
    k_select_reg<4><<<grid, kOneGroup, 0, s>>>(x, n, k, idx_out, x_stride);
  else if (n <= kOneGroup * 16)
    k_select_reg<16><<<grid, kOneGroup, 0, s>>>(x, n, k, idx_out, x_stride);
  else
    k_select<<<grid, kOneGroup, 0, s>>>(x, n, k, idx_out, x_stride);
  return check_launch("k_select");
}

int launch_select(const uint16_t* x, int n, int k, int32_t* idx_out, hipStream_t s) {
  return launch_select_batch(x, n, k, idx_out, 1, n, s);
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
  if (pl.n_splits == 1) return launch_gemv(IN_LIST, OUT_BF16, p, s);
  int rc = launch_gemv(IN_LIST, OUT_PARTIAL, p, s);
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
