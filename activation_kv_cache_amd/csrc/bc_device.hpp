// bc_device.hpp -- device helpers shared by the gfx950 kernels of libbc.
//
// bf16 handling, 64-lane wavefront reductions (DPP within 16-lane rows),
// block-wide scans, the order-preserving float key, and the block-wide exact
// top-k (radix select over integer keys, equal keys by lower position,
// output in ascending position order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bc {

constexpr int kWave = 64;

// ----------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even on the bit pattern (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Order-preserving map float -> uint32 (larger float, larger key; -0 < +0).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// --------------------------------------------------------- DPP reductions
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16

// Sum over groups of W consecutive lanes (W in {4, 8, 16}); every lane of
// the group ends with the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_f<kDppMirror>(v);
  return v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

// Cross-lane shuffles through LDS (ds_bpermute) cost about as much as a
// barrier on this chip; the helpers below use DPP (row operations at VALU
// latency) and v_readlane instead.

// The value of lane (lane ^ OFF), OFF in {8, 16, 32}, without LDS: DPP
// row_ror:8 within 16-lane rows; gfx950's v_permlane16_swap / 32_swap, which
// leave each lane its own value and its partner's in a row-dependent order.
// Other offsets fall back to a shuffle.
template <int OFF>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (OFF == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(((threadIdx.x >> 4) & 1) ? r[0] : r[1]);
  } else if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  } else {
    return __shfl_xor(v, OFF, kWave);
  }
}

// Integer sum over the 64 lanes of a wave; the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u<0xB1>(v);     // xor 1
  v += dpp_u<0x4E>(v);     // xor 2
  v += dpp_u<0x141>(v);    // half mirror: xor 4 on uniform quads
  v += dpp_u<0x140>(v);    // mirror: xor 8 on uniform halves
  return uint32_t(__builtin_amdgcn_readlane(int(v), 0)) + uint32_t(__builtin_amdgcn_readlane(int(v), 16)) +
         uint32_t(__builtin_amdgcn_readlane(int(v), 32)) + uint32_t(__builtin_amdgcn_readlane(int(v), 48));
}

// Float sum over the 64 lanes with a fixed order (row butterflies, then the
// four row sums in row order); the result is wave-uniform.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts within 16-lane
// rows, then row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, true));   // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, true));   // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, true));   // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, true));   // row_shr:8
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15 -> rows 1, 3
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31 -> rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_lane() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = wave_lane();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// ------------------------------------------------------- split partials
// Sum of the n_splits chunk partials of column c, in chunk order.  Up to 8
// chunks are loaded at once (one memory round trip for the usual plans).
// Loads use clamped indices (no branches), so the loads of several
// chunk_sum calls can all be in flight together.
__device__ __forceinline__ float chunk_sum(const float* partial, int n_splits, int d_out, int c) {
  float v = 0.f;
  for (int s = 0; s < n_splits; s += 8) {
    float a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = partial[size_t(min(s + u, n_splits - 1)) * d_out + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) v = s + u < n_splits ? v + a[u] : v;
  }
  return v;
}


// Chunks of q/k/v partials the attention and scoring prologues add (all
// their loads unrolled): the layer's q/k/v GEMV is planned with at most this
// many.
constexpr int kQkvMaxChunks = 8;

// The same sum split in two for at most kQkvMaxChunks chunks, so that
// other loads can be issued between the loads and the sum (memory counters
// retire in order): chunk_load issues the chunk loads, chunk_total adds them
// in chunk order -- the result equals chunk_sum's.  No loop: a loop of loads
// ahead of the sum makes the compiler wait for every load issued so far (the
// first K/V rows or block summaries included) before the sum; the launchers
// reject more chunks.
struct Chunk8 {
  float a[kQkvMaxChunks];
};
__device__ __forceinline__ void chunk_load(Chunk8& c, const float* partial, int n_splits, int d_out, int col) {
#pragma unroll
  for (int u = 0; u < kQkvMaxChunks; ++u) c.a[u] = partial[size_t(min(u, n_splits - 1)) * d_out + col];
}
__device__ __forceinline__ float chunk_total(const Chunk8& c, int n_splits) {
  float v = 0.f;
#pragma unroll
  for (int u = 0; u < kQkvMaxChunks; ++u) v = u < n_splits ? v + c.a[u] : v;
  return v;
}

// ------------------------------------------------------ block top-k select
// Keys are staged in LDS when they fit (kTopkLdsBytes); larger inputs read
// key_fn directly.
constexpr int kTopkLdsBytes = 65536;

template <int NT, typename KeyT>
struct TopkSmem {
  static constexpr int CAP = kTopkLdsBytes / int(sizeof(KeyT));
  KeyT keys[CAP];
  uint32_t hist[NT / kWave][256];
  uint32_t wave_gt[NT / kWave];
  uint32_t wave_eq[NT / kWave];
  uint32_t cnt[2][NT / kWave][8];
  uint32_t scan[NT / kWave + 1];
  uint32_t sel_bin, sel_above;
};

// Keys per thread of the register path of block_topk.
constexpr int kTopkRegKeys = 16;

// Exact top-k when n <= NT * kTopkRegKeys and the keys are in sm.keys
// (synchronised).  Thread t owns positions [t*E, t*E + E), E = ceil(n/NT),
// held in registers.  Radix passes of 4-bit digits from the top: each thread
// counts its keys per digit in packed 8-bit fields (no atomics), the wave
// adds them as 16-bit fields, wave 0 adds the waves and picks the digit.
// Then one block scan of (ties, greater) counts places every kept position:
// the ties kept before thread t are min(ties before t, ties needed).
template <int NT, int BITS, typename KeyT, typename EmitFn>
__device__ void block_topk_reg(int n, int k, EmitFn emit, TopkSmem<NT, KeyT>& sm) {
  constexpr int NW = NT / kWave;
  constexpr int NPASS = (BITS + 3) / 4;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int E = (n + NT - 1) / NT;
  const int i0 = tid * E;
  // positions past n hold key 0 and are excluded by the valid count nv
  const int nv = max(0, min(E, n - i0));
  uint32_t key[kTopkRegKeys];
#pragma unroll
  for (int e = 0; e < kTopkRegKeys; ++e) key[e] = e < nv ? uint32_t(sm.keys[i0 + e]) : 0u;
  uint32_t prefix = 0, k_rem = uint32_t(k);
  int decided = 0;
  const uint32_t keymask = BITS == 32 ? ~0u : ((1u << BITS) - 1u);
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    const int width = (BITS - decided) >= 4 ? 4 : (BITS - decided);
    const int shift = BITS - decided - width;
    const uint32_t hi_mask = decided == 0 ? 0u : ((~0u << (BITS - decided)) & keymask);
    uint64_t c_lo = 0, c_hi = 0;
#pragma unroll
    for (int e = 0; e < kTopkRegKeys; ++e) {
      if (e < nv && ((key[e] ^ prefix) & hi_mask) == 0) {
        const uint32_t d = (key[e] >> shift) & 15u;
        const uint64_t one = 1ull << (8 * (d & 7u));
        if (d < 8) c_lo += one; else c_hi += one;
      }
    }
    // 16 digits as 16-bit fields of 8 words: word i holds digits 2i, 2i+1
    uint32_t* cnt = sm.cnt[pass & 1][w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = uint32_t((c_lo >> (16 * i)) & 0xFF) | (uint32_t((c_lo >> (16 * i + 8)) & 0xFF) << 16);
      const uint32_t hi = uint32_t((c_hi >> (16 * i)) & 0xFF) | (uint32_t((c_hi >> (16 * i + 8)) & 0xFF) << 16);
      const uint32_t slo = wave_sum_u32(lo), shi = wave_sum_u32(hi);
      if (lane == 0) { cnt[i] = slo; cnt[4 + i] = shi; }
    }
    __syncthreads();
    // every wave picks the digit (no second barrier): lane L < 16 owns digit
    // 15 - L, so the lane prefix is the count of keys with larger digits
    const int d = 15 - lane;
    uint32_t c = 0;
    if (lane < 16)
      for (int ww = 0; ww < NW; ++ww) c += (sm.cnt[pass & 1][ww][d >> 1] >> (16 * (d & 1))) & 0xFFFFu;
    const uint32_t inc = wave_scan_dpp(c);
    const uint32_t ex = inc - c;
    const uint64_t hit = __ballot(lane < 16 && ex < k_rem && k_rem <= inc);
    const int hl = __ffsll((long long)hit) - 1;
    const uint32_t sel_d = uint32_t(15 - hl);
    const uint32_t above = uint32_t(__builtin_amdgcn_readlane(int(ex), hl));
    prefix |= sel_d << shift;
    k_rem -= above;
    decided += width;
  }
  const uint32_t thr = prefix, need = k_rem;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kTopkRegKeys; ++e) {
    gt += (e < nv && key[e] > thr) ? 1u : 0u;
    eq += (e < nv && key[e] == thr) ? 1u : 0u;
  }
  // exclusive block scan of (eq << 16 | gt)
  const uint32_t v = (eq << 16) | gt;
  const uint32_t inc = wave_scan_dpp(v);
  if (lane == kWave - 1) sm.scan[w] = inc;
  __syncthreads();
  uint32_t before = inc - v;
  for (int ww = 0; ww < w; ++ww) before += sm.scan[ww];
  const uint32_t gt_before = before & 0xFFFFu, eq_before = before >> 16;
  uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
  uint32_t tie = eq_before;
#pragma unroll
  for (int e = 0; e < kTopkRegKeys; ++e) {
    if (e >= nv) continue;
    if (key[e] > thr) {
      emit(int(pos++), i0 + e);
    } else if (key[e] == thr) {
      if (tie < need) emit(int(pos++), i0 + e);
      ++tie;
    }
  }
  __syncthreads();
}

// Exact top-k over n integer keys given by key_fn(i) (the low BITS bits are
// used; BITS in {15, 32}).  Keeps the k largest keys, equal keys by lower
// position, and calls emit(rank, i) for every kept position, rank being its
// place in ascending position order.  Every thread of the block must call it.
//   1. keys staged in LDS (if they fit);
//   2. radix passes of 8 bits from the top, per-wave histograms, wave 0 finds
//      the bin holding the k-th largest key -> threshold key thr and the
//      number need_eq of keys equal to thr that are kept;
//   3. each wave owns a contiguous slice of positions; per-wave counts of
//      keys > thr and == thr give every wave its tie allowance and output
//      offset; a ballot pass then emits the kept positions in order.
template <int NT, int BITS, typename KeyT, typename KeyFn, typename EmitFn>
__device__ void block_topk(int n, int k, KeyFn key_fn, EmitFn emit, TopkSmem<NT, KeyT>& sm,
                           bool keys_staged = false) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) emit(i, i);
    return;
  }
  if (k <= 0) return;
  // keys_staged: the caller already wrote sm.keys[0..n) and synchronised
  const bool staged = keys_staged || n <= TopkSmem<NT, KeyT>::CAP;
  if (staged && !keys_staged) {
    for (int i = tid; i < n; i += NT) sm.keys[i] = KeyT(key_fn(i));
  }
  if (staged && n <= NT * kTopkRegKeys) {
    if (!keys_staged) __syncthreads();
    block_topk_reg<NT, BITS, KeyT>(n, k, emit, sm);
    return;
  }
  auto key = [&](int i) -> uint32_t { return staged ? uint32_t(sm.keys[i]) : uint32_t(key_fn(i)); };

  uint32_t prefix = 0;
  int decided = 0;
  uint32_t k_rem = uint32_t(k);
  constexpr int NPASS = (BITS + 7) / 8;
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    const int width = (BITS - decided) >= 8 ? 8 : (BITS - decided);
    const int shift = BITS - decided - width;
    const uint32_t keymask = BITS == 32 ? ~0u : ((1u << BITS) - 1u);
    const uint32_t hi_mask = decided == 0 ? 0u : ((~0u << (BITS - decided)) & keymask);
    for (int i = lane; i < 256; i += kWave) sm.hist[w][i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t kk = key(i);
      if (((kk ^ prefix) & hi_mask) == 0) atomicAdd(&sm.hist[w][(kk >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    if (w == 0) {
      // lane owns bins 255-4*lane .. 252-4*lane (descending)
      uint32_t c[4];
      uint32_t sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = 255 - 4 * lane - u;
        uint32_t t = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) t += sm.hist[ww][b];
        c[u] = t;
        sum += t;
      }
      const uint32_t inc = wave_inclusive_scan(sum);
      const uint32_t ex = inc - sum;
      if (ex < k_rem && k_rem <= inc) {
        uint32_t run = ex;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (run < k_rem && k_rem <= run + c[u]) { sm.sel_bin = uint32_t(255 - 4 * lane - u); sm.sel_above = run; }
          run += c[u];
        }
      }
    }
    __syncthreads();
    prefix |= sm.sel_bin << shift;
    k_rem -= sm.sel_above;
    decided += width;
  }
  const uint32_t thr = prefix, need_eq = k_rem;

  // per-wave counts over its contiguous slice
  const int per = (n + NW - 1) / NW;
  const int w0 = min(n, w * per), w1 = min(n, w0 + per);
  uint32_t gt = 0, eq = 0;
  for (int b = w0; b < w1; b += kWave) {
    const int i = b + lane;
    const uint32_t kk = i < w1 ? key(i) : 0u;
    const bool in = i < w1;
    gt += __popcll(__ballot(in && kk > thr));
    eq += __popcll(__ballot(in && kk == thr));
  }
  if (lane == 0) { sm.wave_gt[w] = gt; sm.wave_eq[w] = eq; }
  __syncthreads();
  uint32_t eq_before = 0, out = 0;
  for (int ww = 0; ww < w; ++ww) {
    const uint32_t e = sm.wave_eq[ww];
    const uint32_t allow = eq_before >= need_eq ? 0u : min(e, need_eq - eq_before);
    out += sm.wave_gt[ww] + allow;
    eq_before += e;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b = w0; b < w1; b += kWave) {
    const int i = b + lane;
    const bool in = i < w1;
    const uint32_t kk = in ? key(i) : 0u;
    const uint64_t eqm = __ballot(in && kk == thr);
    const uint32_t my_tie = eq_before + uint32_t(__popcll(eqm & below));
    const bool take = in && (kk > thr || (kk == thr && my_tie < need_eq));
    const uint64_t tm = __ballot(take);
    if (take) emit(int(out + uint32_t(__popcll(tm & below))), i);
    out += uint32_t(__popcll(tm));
    eq_before += uint32_t(__popcll(eqm));
  }
  __syncthreads();
}

// ---------------------------------------------------- split-K combine
// The fp32 order in which one head's split partials (m in natural-log units,
// l, unnormalised o; S splits) are combined.  k_attn_reduce and the o GEMV
// prologue that folds the reduce in both follow it, so both give the same
// bf16 attention output:
//   M = max_s m_s;  w_s = exp(m_s - M), or 0 when m_s or M is -inf;
//   den: thread t of kCombineThreads sums w_s l_s over s = t, t + 256, ...
//        in order (fmaf from 0), each wave's sum is wave_sum_f32's (DPP
//        pairs, quads, eights and sixteens within each row of 16 lanes, then
//        the four rows as (r0 + r1) + (r2 + r3)), and the wave sums are added
//        in order to 0;
//   num_d: G = kCombineThreads / D groups of ceil(S / G) consecutive splits,
//        each summed in split order with fmaf from 0 (combine_group), the
//        group sums added in order to 0;
//   out_d = bf16(den > 0 ? num_d / den : 0).
constexpr int kCombineThreads = 256;

__device__ __forceinline__ float combine_weight(float ms, float M) {
  return (ms == -INFINITY || M == -INFINITY) ? 0.f : expf(ms - M);
}

// splits [s0, s1) of one group; o(s) and w(s) give o_s[d] and w_s
template <typename OF, typename WF>
__device__ __forceinline__ float combine_group(int s0, int s1, OF o, WF w) {
  float num = 0.f;
#pragma unroll 4
  for (int s = s0; s < s1; ++s) num = fmaf(o(s), w(s), num);
  return num;
}

__device__ __forceinline__ float combine_wave_sum(float v) { return wave_sum_f32(v); }

// Largest value over the 64 lanes (exact in any order): DPP within rows of
// 16, then the four rows.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ------------------------------------- 15-bit keys in registers, two passes
// Exact top-k of n keys below 2^15 held in registers by NT threads: thread t
// owns positions [t*P, t*P + P) (positions >= n are ignored), so a thread's
// keys are in position order.  Pass 1 histograms the top 15-SHIFT key bits
// (LDS atomics); the bin holding the k-th largest key is found from per-wave
// totals and a scan inside the one wave whose bins cross k.  Pass 2
// histograms the low SHIFT bits of the keys in that bin.  That fixes the
// threshold key thr and the number `need` of keys equal to thr that are kept
// (the lowest positions).  One block scan of (ties, greater) counts per
// thread gives each thread the rank of its first kept key; ranks within the
// thread come from popcounts of the kept-key bit mask, so no thread walks its
// keys serially.  emit(rank - r0, e) is called for the thread's e-th key when
// it is kept and its rank is in [r0, r1); with `all`, out(rank, e) is also
// called for every kept key.
//
// All NT threads execute every instruction of the block-wide steps, so the
// searches over wave totals and over the low digit run lane-parallel (one
// value per lane, a 16-lane DPP scan, a ballot) instead of as per-thread
// loops.  The caller zeroes the histogram with topk2_clear() and passes a
// __syncthreads() before the call (so the clear can overlap its own loads).
// Requires 1 <= k <= n <= NT * PMAX, PMAX <= 32, NT <= 16 waves, n < 65536
// (the rank scan packs two 16-bit counts).  Contains __syncthreads(); the
// caller synchronises before reading what emit wrote.
template <int NT, int SHIFT>
struct Topk2Smem {
  static constexpr int NB = 32768 >> SHIFT;
  uint32_t hist[NB];
  uint32_t hist2[1 << SHIFT];
  uint32_t wtot[NT / kWave];
  uint32_t b1, above1;
};

template <int NT, int SHIFT>
__device__ __forceinline__ void topk2_clear(Topk2Smem<NT, SHIFT>& sm) {
  constexpr int NQ = Topk2Smem<NT, SHIFT>::NB / 4;
  static_assert(NQ % NT == 0, "whole uint4 of bins per thread");
  uint4* h4 = reinterpret_cast<uint4*>(sm.hist);
#pragma unroll
  for (int i = 0; i < NQ / NT; ++i) h4[threadIdx.x + i * NT] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x < (1 << SHIFT)) sm.hist2[threadIdx.x] = 0u;
}

// Inclusive prefix sum within each 16-lane row.
__device__ __forceinline__ uint32_t row16_scan(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, true));   // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, true));   // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, true));   // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, true));   // row_shr:8
  return v;
}

// Sum of wave totals tot[0..w) for the calling wave w (w uniform, NW <= 16):
// lane l holds tot[l], one row scan, one readlane.
template <int NW>
__device__ __forceinline__ uint32_t waves_before(const uint32_t* tot, int w) {
  static_assert(NW <= 16, "one DPP row");
  const int lane = threadIdx.x & 63;
  const uint32_t inc = row16_scan(lane < NW ? tot[lane] : 0u);
  return w == 0 ? 0u : uint32_t(__builtin_amdgcn_readlane(int(inc), w - 1));
}

// Sum of wave totals tot[0..w) and of all NW of them, lane-parallel.
template <int NW>
__device__ __forceinline__ void waves_before_total(const uint32_t* tot, int w, uint32_t* before, uint32_t* total) {
  static_assert(NW <= 16, "one DPP row");
  const int lane = threadIdx.x & 63;
  const uint32_t inc = row16_scan(lane < NW ? tot[lane] : 0u);
  *before = w == 0 ? 0u : uint32_t(__builtin_amdgcn_readlane(int(inc), w - 1));
  *total = uint32_t(__builtin_amdgcn_readlane(int(inc), NW - 1));
}

// Emission of one thread's kept keys: the i-th set bit of `take` (low bits
// first) holds rank pos0 + i.  emit(rank - r0, e) for ranks in [r0, r1), one
// popcount, compare and store per key and no branch but the store's own;
// with `all`, out(rank, e) for every kept key.  Threads whose ranks miss
// [r0, r1) skip the loop.
struct TopkNoOut {
  __device__ void operator()(int, int) const {}
};
// stamp(i) after the selection's i-th barrier (i = 0..4) and at its end (5)
struct TopkNoStamp {
  __device__ void operator()(int) const {}
};

template <int PMAX, typename EmitFn, typename OutFn>
__device__ __forceinline__ void topk_emit_kept(uint32_t take, uint32_t pos0, uint32_t cnt, int r0, int r1, bool all,
                                               EmitFn& emit, OutFn& out) {
  if (all) {
#pragma unroll
    for (int e = 0; e < PMAX; ++e)
      if ((take >> e) & 1u) out(int(pos0 + uint32_t(__popc(take & ((1u << e) - 1u)))), e);
  }
  if (pos0 < uint32_t(r1) && pos0 + cnt > uint32_t(r0)) {
    const uint32_t span = uint32_t(r1 - r0);
    const uint32_t rel0 = pos0 - uint32_t(r0);   // wraps below r0: those ranks fail rel < span
#pragma unroll
    for (int e = 0; e < PMAX; ++e) {
      const uint32_t rel = rel0 + uint32_t(__popc(take & ((1u << e) - 1u)));
      if (((take >> e) & 1u) && rel < span) emit(int(rel), e);
    }
  }
}

template <int NT, int SHIFT, int PMAX, typename EmitFn, typename OutFn = TopkNoOut, typename StampFn = TopkNoStamp>
__device__ void block_topk_2pass(const uint32_t (&key)[PMAX], int P, int n, int k, int r0, int r1, EmitFn emit,
                                 Topk2Smem<NT, SHIFT>& sm, bool all = false, OutFn out = OutFn(),
                                 StampFn stamp = StampFn()) {
  static_assert(PMAX <= 32, "bit masks are 32 bits");
  constexpr int NB = Topk2Smem<NT, SHIFT>::NB;
  constexpr int NB2 = 1 << SHIFT;
  static_assert(NB2 <= 16, "low digit found in one DPP row");
  constexpr int NW = NT / kWave;
  static_assert(NW <= 16, "wave totals found in one DPP row");
  constexpr int BPT = NB / NT;  // bins per thread
  static_assert(BPT % 4 == 0, "whole uint4 of bins per thread");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nv = max(0, min(P, n - tid * P));
  const uint32_t ku = uint32_t(k);
#pragma unroll
  for (int e = 0; e < PMAX; ++e) {
    const bool ok = e < nv;
    atomicAdd(&sm.hist[ok ? key[e] >> SHIFT : uint32_t(lane)], ok ? 1u : 0u);
  }
  __syncthreads();
  stamp(0);
  // thread t owns bins [b0, b0 + BPT), b0 = NB - BPT (t + 1): the largest
  // bins go to thread 0, so counts accumulated over threads in order count
  // larger keys
  const int b0 = NB - BPT * (tid + 1);
  uint32_t bins[BPT];
  uint32_t local = 0;
  {
    const uint4* hb = reinterpret_cast<const uint4*>(sm.hist + b0);
#pragma unroll
    for (int q = 0; q < BPT / 4; ++q) {
      const uint4 c = hb[q];
      bins[4 * q] = c.x; bins[4 * q + 1] = c.y; bins[4 * q + 2] = c.z; bins[4 * q + 3] = c.w;
      local += (c.x + c.y) + (c.z + c.w);
    }
  }
  const uint32_t winc = wave_scan_dpp(local);
  if (lane == kWave - 1) sm.wtot[w] = winc;
  __syncthreads();
  stamp(1);
  {
    // the wave whose bins hold the k-th largest key (lane-parallel search)
    const uint32_t c = lane < NW ? sm.wtot[lane] : 0u;
    const uint32_t inc = row16_scan(c), ex = inc - c;
    const uint64_t hitw = __ballot(lane < NW && ex < ku && ku <= inc);
    const int ws = __ffsll((long long)hitw) - 1;
    if (w == ws) {
      const uint32_t above_w = uint32_t(__builtin_amdgcn_readlane(int(ex), ws));
      const uint32_t tinc = above_w + winc, tex = tinc - local;
      if (tex < ku && ku <= tinc) {
        uint32_t run = tex;
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
          if (run < ku && ku <= run + bins[j]) { sm.b1 = uint32_t(b0 + j); sm.above1 = run; }
          run += bins[j];
        }
      }
    }
  }
  __syncthreads();
  stamp(2);
  const uint32_t b1 = sm.b1, k2 = ku - sm.above1;
#pragma unroll
  for (int e = 0; e < PMAX; ++e)
    if (e < nv && (key[e] >> SHIFT) == b1) atomicAdd(&sm.hist2[key[e] & uint32_t(NB2 - 1)], 1u);
  __syncthreads();
  stamp(3);
  uint32_t thr, need;
  {
    // low digit, largest first: lane l holds digit NB2-1-l
    const uint32_t c = lane < NB2 ? sm.hist2[NB2 - 1 - lane] : 0u;
    const uint32_t inc = row16_scan(c), ex = inc - c;
    const uint64_t hit = __ballot(lane < NB2 && ex < k2 && k2 <= inc);
    const int hl = __ffsll((long long)hit) - 1;
    thr = (b1 << SHIFT) | uint32_t(NB2 - 1 - hl);
    need = k2 - uint32_t(__builtin_amdgcn_readlane(int(ex), hl));
  }
  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int e = 0; e < PMAX; ++e) {
    if (e < nv) {
      gtm |= (key[e] > thr ? 1u : 0u) << e;
      eqm |= (key[e] == thr ? 1u : 0u) << e;
    }
  }
  const uint32_t gt = uint32_t(__popc(gtm)), eq = uint32_t(__popc(eqm));
  // exclusive block scan of (eq << 16 | gt); wtot is free again (its last
  // readers passed two barriers ago)
  const uint32_t v = (eq << 16) | gt;
  const uint32_t inc = wave_scan_dpp(v);
  if (lane == kWave - 1) sm.wtot[w] = inc;
  __syncthreads();
  stamp(4);
  const uint32_t bf = inc - v + waves_before<NW>(sm.wtot, w);
  const uint32_t gt_before = bf & 0xFFFFu, eq_before = bf >> 16;
  const uint32_t ties_before = eq_before < need ? eq_before : need;
  const uint32_t ties_here = (eq_before + eq < need ? eq_before + eq : need) - ties_before;
  // keep the lowest ties_here of the thread's ties
  uint32_t tie_keep = eqm;
  if (ties_here < eq) {
    tie_keep = 0;
    uint32_t m = eqm;
    for (uint32_t i = 0; i < ties_here; ++i) {
      const uint32_t low = m & (~m + 1u);
      tie_keep |= low;
      m ^= low;
    }
  }
  topk_emit_kept<PMAX>(gtm | tie_keep, gt_before + ties_before, gt + ties_here, r0, r1, all, emit, out);
  stamp(5);
}

// --------------------------------------- 32-bit keys in registers, adaptive
// Exact top-k of n 32-bit keys held in registers by NT threads, thread t
// owning positions [t*P, t*P + P) (positions >= n ignored); ties go to the
// lower position.  Order-preserving keys of fp32 scores crowd into a few
// exponents, so the first histogram is taken over the keys' own range:
// bins (key - min) >> shift, 2048 of them (LDS atomics rarely collide then).
// Later passes resolve the chosen bin 13 bits at a time (8192 bins) until
// the threshold key thr is exact; the number `need` of keys equal to thr
// that are kept follows.  The ranks come from one block scan of (ties,
// greater) and per-thread popcounts, as in block_topk_2pass; emit(rank - r0,
// e) for kept keys whose rank is in [r0, r1).
// Requires 1 <= k <= n <= NT * PMAX, PMAX <= 32, n < 65536.  Contains
// __syncthreads(); the caller synchronises before reading what emit wrote.
template <int NT>
struct Topk32Smem {
  static constexpr int kCandCap = 256;   // keys of the chosen bin ranked by brute force
  uint32_t hist[8192];
  uint32_t cand[kCandCap];
  uint32_t wlo[NT / kWave];
  uint32_t whi[NT / kWave];
  uint32_t sel_bin, sel_above;
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<0xB1>(v));
  v = min(v, dpp_u<0x4E>(v));
  v = min(v, dpp_u<0x141>(v));
  v = min(v, dpp_u<0x140>(v));
  const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int(v), 0)), b = uint32_t(__builtin_amdgcn_readlane(int(v), 16));
  const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(v), 32)), d = uint32_t(__builtin_amdgcn_readlane(int(v), 48));
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int(v), 0)), b = uint32_t(__builtin_amdgcn_readlane(int(v), 16));
  const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(v), 32)), d = uint32_t(__builtin_amdgcn_readlane(int(v), 48));
  return max(max(a, b), max(c, d));
}

// One histogram pass: bins hist[0..NB) hold counts of the keys in range;
// finds the bin holding the k_rem-th largest of them (bins taken from the
// top) and stores it with the count above it in sm.sel_bin / sm.sel_above.
template <int NT, int NB>
__device__ __forceinline__ void topk32_pick_bin(uint32_t k_rem, Topk32Smem<NT>& sm) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = NB / NT;
  static_assert(BPT >= 1 && NB % NT == 0, "bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b0 = NB - BPT * (tid + 1);
  uint32_t bins[BPT];
  uint32_t local = 0;
  if constexpr (BPT % 4 == 0) {
    // neighbouring threads' ranges are BPT words apart: read the 16-byte
    // pieces in a thread-rotated order so the lanes spread over the banks
    constexpr int NQ = BPT / 4;
    const uint4* hb = reinterpret_cast<const uint4*>(sm.hist + b0);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int jj = (j + tid) % NQ;
      const uint4 c = hb[jj];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q == jj) { bins[4 * q] = c.x; bins[4 * q + 1] = c.y; bins[4 * q + 2] = c.z; bins[4 * q + 3] = c.w; }
      }
      local += (c.x + c.y) + (c.z + c.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      bins[j] = sm.hist[b0 + j];
      local += bins[j];
    }
  }
  const uint32_t winc = wave_scan_dpp(local);
  if (lane == kWave - 1) sm.whi[w] = winc;
  __syncthreads();
  const uint32_t before = waves_before<NW>(sm.whi, __builtin_amdgcn_readfirstlane(w));
  const uint32_t inc = before + winc, ex = inc - local;
  if (ex < k_rem && k_rem <= inc) {
    uint32_t run = ex;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (run < k_rem && k_rem <= run + bins[j]) { sm.sel_bin = uint32_t(b0 + j); sm.sel_above = run; }
      run += bins[j];
    }
  }
  __syncthreads();
}

template <int NT, int PMAX, typename EmitFn>
__device__ void block_topk32(const uint32_t (&key)[PMAX], int P, int n, int k, int r0, int r1, EmitFn emit,
                             Topk32Smem<NT>& sm) {
  const bool all = false;
  TopkNoOut out;
  static_assert(PMAX <= 32, "bit masks are 32 bits");
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nv = max(0, min(P, n - tid * P));
  // key range; the first histogram is cleared under the same barrier
  uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
  for (int e = 0; e < PMAX; ++e)
    if (e < nv) { kmin = min(kmin, key[e]); kmax = max(kmax, key[e]); }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) { sm.wlo[w] = kmin; sm.whi[w] = kmax; }
  {
    uint4* h4 = reinterpret_cast<uint4*>(sm.hist);
    for (int i = tid; i < 2048 / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  // every wave reduces the wave minima and maxima itself, one per lane
  kmin = wave_min_u32(lane < NW ? sm.wlo[lane] : ~0u);
  kmax = wave_max_u32(lane < NW ? sm.whi[lane] : 0u);
  const uint32_t range = kmax - kmin;
  const int shift = range == 0u ? 0 : max(0, 32 - __clz(int(range)) - 11);   // (range >> shift) < 2048
  __syncthreads();   // whi is reused by the scans
  // every lane adds: positions past n add 0 into a bin of their own lane
  // (no branches and no colliding dummy adds)
#pragma unroll
  for (int e = 0; e < PMAX; ++e) {
    const bool ok = e < nv;
    atomicAdd(&sm.hist[ok ? (key[e] - kmin) >> shift : uint32_t(lane)], ok ? 1u : 0u);
  }
  __syncthreads();
  topk32_pick_bin<NT, 2048>(uint32_t(k), sm);
  const uint32_t b1 = sm.sel_bin;
  uint32_t base = kmin + (b1 << shift);
  uint32_t k_rem = uint32_t(k) - sm.sel_above;
  int rem_bits = shift;
  if (rem_bits > 0) {
    // the chosen bin usually holds a few keys: gather them and rank each by
    // brute force (larger keys, then equal keys); the one whose rank span
    // holds k_rem is the threshold
    uint32_t inb = 0;
#pragma unroll
    for (int e = 0; e < PMAX; ++e) inb |= (e < nv && ((key[e] - kmin) >> shift) == b1 ? 1u : 0u) << e;
    // slots by a block scan of the per-thread counts (no returning atomics)
    const uint32_t cnt = uint32_t(__popc(inb));
    const uint32_t cinc = wave_scan_dpp(cnt);
    if (lane == kWave - 1) sm.whi[w] = cinc;
    __syncthreads();
    uint32_t off, nc;
    waves_before_total<NW>(sm.whi, __builtin_amdgcn_readfirstlane(w), &off, &nc);
    off += cinc - cnt;
    if (inb != 0u && off < uint32_t(Topk32Smem<NT>::kCandCap)) {
#pragma unroll
      for (int e = 0; e < PMAX; ++e) {
        if ((inb >> e) & 1u) {
          const uint32_t slot = off + uint32_t(__popc(inb & ((1u << e) - 1u)));
          if (slot < uint32_t(Topk32Smem<NT>::kCandCap)) sm.cand[slot] = key[e];
        }
      }
    }
    __syncthreads();
    if (nc <= uint32_t(Topk32Smem<NT>::kCandCap)) {
      for (uint32_t t = uint32_t(tid); t < nc; t += NT) {
        const uint32_t v = sm.cand[t];
        uint32_t gt = 0, eq = 0;
        for (uint32_t j = 0; j < nc; ++j) {
          const uint32_t c = sm.cand[j];
          gt += c > v ? 1u : 0u;
          eq += c == v ? 1u : 0u;
        }
        if (gt < k_rem && k_rem <= gt + eq) { sm.sel_bin = v; sm.sel_above = gt; }   // equal v write equal values
      }
      __syncthreads();
      base = sm.sel_bin;
      k_rem -= sm.sel_above;
      rem_bits = 0;
    }
  }
  while (rem_bits > 0) {   // crowded bin: radix passes (uniform over the work-group)
    const int wbits = min(13, rem_bits);
    const int sh = rem_bits - wbits;
    {
      uint4* h4 = reinterpret_cast<uint4*>(sm.hist);
      for (int i = tid; i < 8192 / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    const uint32_t span = rem_bits >= 32 ? ~0u : ((1u << rem_bits) - 1u);
#pragma unroll
    for (int e = 0; e < PMAX; ++e)
      if (e < nv && key[e] >= base && key[e] - base <= span) atomicAdd(&sm.hist[(key[e] - base) >> sh], 1u);
    __syncthreads();
    topk32_pick_bin<NT, 8192>(k_rem, sm);
    base += sm.sel_bin << sh;
    k_rem -= sm.sel_above;
    rem_bits = sh;
  }
  const uint32_t thr = base, need = k_rem;
  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int e = 0; e < PMAX; ++e) {
    if (e < nv) {
      gtm |= (key[e] > thr ? 1u : 0u) << e;
      eqm |= (key[e] == thr ? 1u : 0u) << e;
    }
  }
  const uint32_t gt = uint32_t(__popc(gtm)), eq = uint32_t(__popc(eqm));
  const uint32_t v = (eq << 16) | gt;
  const uint32_t inc = wave_scan_dpp(v);
  if (lane == kWave - 1) sm.whi[w] = inc;
  __syncthreads();
  const uint32_t bf = inc - v + waves_before<NW>(sm.whi, __builtin_amdgcn_readfirstlane(w));
  const uint32_t gt_before = bf & 0xFFFFu, eq_before = bf >> 16;
  const uint32_t ties_before = eq_before < need ? eq_before : need;
  const uint32_t ties_here = (eq_before + eq < need ? eq_before + eq : need) - ties_before;
  uint32_t tie_keep = eqm;
  if (ties_here < eq) {
    tie_keep = 0;
    uint32_t m = eqm;
    for (uint32_t i = 0; i < ties_here; ++i) {
      const uint32_t low = m & (~m + 1u);
      tie_keep |= low;
      m ^= low;
    }
  }
  topk_emit_kept<PMAX>(gtm | tie_keep, gt_before + ties_before, gt + ties_here, r0, r1, all, emit, out);
}

// Keys of n fp32 scores for block_topk32, thread t owning positions
// [t*PMAX, t*PMAX + PMAX) (P = PMAX, so n <= NT*PMAX; positions >= n carry
// don't-care keys that block_topk32 ignores): the scores are read with
// coalesced loads into `stage` (LDS, NT*PMAX words), then each thread takes
// its PMAX keys as 16-byte pieces in a thread-rotated order (the threads'
// ranges are PMAX words apart).  Every index is clamped instead of tested,
// so the code has no branches.  Returns P.  Contains __syncthreads().
template <int NT, int PMAX>
__device__ int load_score_keys(const float* src, int n, uint32_t (&key)[PMAX], uint32_t* stage) {
  static_assert(PMAX % 4 == 0 && ((PMAX / 4) & (PMAX / 4 - 1)) == 0, "power-of-two count of 16-byte pieces");
  constexpr int NQ = PMAX / 4;
  const int tid = threadIdx.x;
  const int last = max(n - 1, 0);
  float v[PMAX];
#pragma unroll
  for (int j = 0; j < PMAX; ++j) v[j] = src[min(tid + j * NT, last)];
#pragma unroll
  for (int j = 0; j < PMAX; ++j) stage[tid + j * NT] = float_order_key(v[j]);
  __syncthreads();
  const uint4* sp = reinterpret_cast<const uint4*>(stage + tid * PMAX);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int jj = (j + tid) & (NQ - 1);
    const uint4 c = sp[jj];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const bool hit = q == jj;
      key[4 * q] = hit ? c.x : key[4 * q];
      key[4 * q + 1] = hit ? c.y : key[4 * q + 1];
      key[4 * q + 2] = hit ? c.z : key[4 * q + 2];
      key[4 * q + 3] = hit ? c.w : key[4 * q + 3];
    }
  }
  __syncthreads();
  return PMAX;
}

}  // namespace bc
