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
// LDS needed by block_topk: NW*256 histogram words + 256 merged + small.
template <int NT>
struct TopkSmem {
  uint32_t hist[NT / kWave][256];
  uint32_t merged[256];
  uint32_t scan[NT / kWave + 1];
  uint32_t sel_bin, sel_above;
};

// Exact top-k over n integer keys given by key_fn(i) (only the low `bits`
// bits are used; bits in {15, 32}).  Keeps the k largest keys, equal keys
// by lower position, and calls emit(rank, i) for every kept position, rank
// being its place in ascending position order.  Every thread of the block
// must call it.  Passes of 8 bits from the top; per-wave histograms in LDS.
template <int NT, int BITS, typename KeyFn, typename EmitFn>
__device__ void block_topk(int n, int k, KeyFn key_fn, EmitFn emit, TopkSmem<NT>& sm) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) emit(i, i);
    return;
  }
  if (k <= 0) return;

  uint32_t prefix = 0;     // decided high bits of the threshold key
  int decided = 0;         // number of decided high bits
  uint32_t k_rem = uint32_t(k);
  int pass_bits[4];
  int npass = 0;
  {
    int left = BITS;
    while (left > 0) { int b = left >= 8 ? 8 : left; pass_bits[npass++] = b; left -= b; }
  }
  for (int p = 0; p < npass; ++p) {
    const int width = pass_bits[p];
    const int shift = BITS - decided - width;
    const uint32_t hi_mask = decided == 0 ? 0u : (~0u << (BITS - decided)) & (BITS == 32 ? ~0u : ((1u << BITS) - 1u));
    for (int i = tid; i < NW * 256; i += NT) (&sm.hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      uint32_t key = key_fn(i);
      if (((key ^ prefix) & hi_mask) == 0)
        atomicAdd(&sm.hist[w][(key >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    for (int b = tid; b < 256; b += NT) {
      uint32_t s = 0;
      for (int ww = 0; ww < NW; ++ww) s += sm.hist[ww][b];
      sm.merged[b] = s;
    }
    __syncthreads();
    if (w == 0) {
      // lane l owns bins 255-4l .. 252-4l (descending); find where the running
      // count from the top reaches k_rem.
      const int lane = wave_lane();
      uint32_t c[4];
      uint32_t s = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { c[u] = sm.merged[255 - 4 * lane - u]; s += c[u]; }
      uint32_t inc = wave_inclusive_scan(s);
      uint32_t ex = inc - s;
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
    __syncthreads();
  }
  // threshold key = prefix; keep every key above it and the first k_rem equal ones.
  const uint32_t thr = prefix;
  const uint32_t need_eq = k_rem;
  const int per = (n + NT - 1) / NT;
  const int i0 = tid * per;
  const int i1 = min(n, i0 + per);
  uint32_t eq = 0;
  for (int i = i0; i < i1; ++i) eq += key_fn(i) == thr;
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan<NT>(eq, sm.scan, &tot);
  uint32_t sel = 0;
  {
    uint32_t e = eq_before;
    for (int i = i0; i < i1; ++i) {
      uint32_t key = key_fn(i);
      if (key > thr) ++sel;
      else if (key == thr) { if (e < need_eq) ++sel; ++e; }
    }
  }
  uint32_t rank = block_exclusive_scan<NT>(sel, sm.scan, &tot);
  {
    uint32_t e = eq_before;
    for (int i = i0; i < i1; ++i) {
      uint32_t key = key_fn(i);
      bool take = false;
      if (key > thr) take = true;
      else if (key == thr) { take = e < need_eq; ++e; }
      if (take) emit(int(rank++), i);
    }
  }
  __syncthreads();
}

}  // namespace bc
