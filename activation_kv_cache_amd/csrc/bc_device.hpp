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

// Block-wide exclusive prefix sum of one value per thread; returns the
// thread's exclusive prefix and writes the block total to *total.
// scratch must hold NT/64 + 1 uint32 in LDS.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int lane = wave_lane(), w = threadIdx.x >> 6;
  uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < NW; ++i) { uint32_t t = scratch[i]; scratch[i] = run; run += t; }
    scratch[NW] = run;
  }
  __syncthreads();
  uint32_t ex = scratch[w] + inc - v;
  *total = scratch[NW];
  __syncthreads();
  return ex;
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
  uint32_t sel_bin, sel_above;
};

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
__device__ void block_topk(int n, int k, KeyFn key_fn, EmitFn emit, TopkSmem<NT, KeyT>& sm) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) emit(i, i);
    return;
  }
  if (k <= 0) return;
  const bool staged = n <= TopkSmem<NT, KeyT>::CAP;
  if (staged) {
    for (int i = tid; i < n; i += NT) sm.keys[i] = KeyT(key_fn(i));
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

}  // namespace bc
