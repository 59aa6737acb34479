// bc_gemv_batch.hip -- batched sparse GEMV with a union channel keep, gfx950.
//
// README "Quick start" (crossover_batch): a batch of sequences reads the
// projection weights once for the union of the channels its sequences keep,
// while the key-value bytes are paid per sequence.  Here sequence b keeps its
// own channel list S_b and gets its own sparse GEMV,
//   y_b = sum over i in S_b of W^T[i] x_b[i],
// and the matrix rows read are those of U = union of the S_b, each once.
//
// One work-group of 1024 lanes per (128-column tile, range of input
// channels).  The prologue forms the work-group's share of U itself: it loads
// the sequences' inputs over its channel range and all list entries, sets a
// bit per (sequence, kept channel of the range) in LDS, ORs the bits into U,
// and compacts U's rows (ascending, as element offsets) with their masked
// inputs x_b[U_j] if U_j is in S_b else 0 (fp32) into LDS.  The row loop then
// streams U's rows like k_gemv: 64 row slots of 16 lanes, a lane loading 16
// bytes (8 columns) of a row and updating the B sequences' sums of its 8
// columns (fp32 multiply-adds).  Chunks are channel ranges, so the launch
// plan needs no count from the device.
#include "bc_device.hpp"
#include "bc_internal.hpp"

namespace bc {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBatchMax = 4;             // sequences per call (more would spill registers)
constexpr int kBatchMaxIn = 16384;       // d_in
constexpr int kBatchRange = 4096;        // input channels per work-group at most
constexpr int kRangeWords = kBatchRange / 32;
constexpr int kPerThread = kBatchRange / kGemvThreads;   // 4: one 8-byte input load per sequence
static_assert(kPerThread == 4, "the vector input load covers four channels");
constexpr int kMaskCopies = 4;                             // copies of each bitmap word (atomic collisions)
constexpr int kRingB = 2;                                  // rows in flight per slot
constexpr int kBatchPad = kBatchRange + 64 * kRingB;       // U's rows + the ring's overrun
constexpr int kSlotsB = kGemvThreads / 16;
constexpr int kNWB = kGemvThreads / kWave;

struct BatchParams {
  const uint16_t* wt;
  int tiled;
  int d_in, d_out, k, nb;
  const uint16_t* x;      // [nb][d_in]
  const int32_t* idx;     // [nb][k] or NULL (every channel)
  int range, n_splits;    // channels per work-group (a multiple of 32), ranges
  int32_t* counts;        // [n_splits] rows of U per range (workspace)
  int32_t* count_out;     // optional |U|
  float* partial;         // [n_splits][nb][d_out] when n_splits > 1
  uint16_t* y;            // [nb][d_out] bf16, or
  float* yf;              // [nb][d_out] fp32 (when y is NULL)
};

struct BatchPlan {
  int n_tiles, n_splits, range;
  size_t off_part, bytes;
};

BatchPlan plan_batch(int d_in, int d_out, int nb) {
  BatchPlan pl{};
  pl.n_tiles = ceil_div(d_out, kGemvTile);
  int splits = (256 + pl.n_tiles / 2) / pl.n_tiles;
  splits = min(splits, max(1, d_in / 64));
  splits = max(splits, 1);
  splits = max(splits, ceil_div(d_in, kBatchRange));
  int range = ceil_div(d_in, splits);
  range = (range + 31) / 32 * 32;
  pl.range = min(range, kBatchRange);
  pl.n_splits = ceil_div(d_in, pl.range);
  pl.off_part = align_up(size_t(pl.n_splits) * 4, 256);
  pl.bytes = pl.off_part + (pl.n_splits > 1 ? align_up(size_t(pl.n_splits) * nb * d_out * 4, 256) : 0);
  return pl;
}

template <int NB>
struct BatchSmem {
  alignas(16) uint32_t mask4[NB][kRangeWords * kMaskCopies];   // S_b over the range, four copies per word
  uint32_t mask[NB][kRangeWords];   // S_b over the range
  uint32_t umask[kRangeWords];      // U over the range
  uint32_t pre[kRangeWords];        // rows of U before each word
  uint32_t wtot[kNWB];
  uint32_t off[kBatchPad];          // U's rows (ascending) as element offsets, padding last
  float4 xf[kBatchPad];             // their masked inputs in fp32 (0 in the padding)
  float red[kNWB][2][NB][kGemvTile];   // per half-wave column sums
};

template <int NB>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_batch(const BatchParams p) {
  __shared__ BatchSmem<NB> sm;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = tid & 15, slot = tid >> 4;
  const int c0 = split * p.range;
  const int c1 = min(p.d_in, c0 + p.range);
  const int nw = (c1 - c0 + 31) / 32;
  const int tile_w = min(kGemvTile, p.d_out - tile * kGemvTile);

  // ------------------------------------------------------------ prologue
  // the inputs of the range first (thread t owns channels c0 + 4t .. 4t + 3:
  // one 8-byte load per sequence when the rows allow it), then the list
  // entries; both are in flight while the bitmaps are cleared
  uint32_t xv[NB][kPerThread];
  const int cq = c0 + kPerThread * tid;
  const bool vec = ((p.d_in & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.x) & 7) == 0);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint16_t* xr = p.x + size_t(b) * p.d_in;
    if (vec && cq + kPerThread <= c1) {
      const uint2 v = *reinterpret_cast<const uint2*>(xr + cq);
      xv[b][0] = v.x & 0xFFFFu; xv[b][1] = v.x >> 16; xv[b][2] = v.y & 0xFFFFu; xv[b][3] = v.y >> 16;
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) xv[b][i] = cq + i < c1 ? uint32_t(xr[cq + i]) : 0u;
    }
  }
  for (int i = tid; i < NB * kRangeWords * kMaskCopies; i += kGemvThreads) (&sm.mask4[0][0])[i] = 0u;
  __syncthreads();
  if (p.idx) {
    // ids outside [0, d_in) are dropped; only the range's ids set bits.
    // Eight entries per thread are loaded before any is used (one memory
    // round trip per pass).  An ascending list puts about 16 consecutive
    // entries in one word, so the bits go to four copies of each word (by
    // lane & 3, adjacent banks) to cut the LDS atomic collisions fourfold.
    const int total_e = NB * p.k;
    const int cp = tid & (kMaskCopies - 1);
    for (int e0 = 0; e0 < total_e; e0 += 8 * kGemvThreads) {
      int cv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + tid + kGemvThreads * u;
        cv[u] = e < total_e ? p.idx[e] : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + tid + kGemvThreads * u;
        const int c = cv[u];
        if (e < total_e && c >= c0 && c < c1)
          atomicOr(&sm.mask4[e / p.k][((c - c0) >> 5) * kMaskCopies + cp], 1u << ((c - c0) & 31));
      }
    }
  } else {
    for (int i = tid; i < NB * nw; i += kGemvThreads) {
      const int b = i / nw, wd = i % nw;
      const int left = c1 - c0 - 32 * wd;
      sm.mask4[b][wd * kMaskCopies] = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
    }
  }
  __syncthreads();
  // U per word and the exclusive prefix of its counts (word order)
  uint32_t cnt = 0;
  if (tid < nw) {
    uint32_t u = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint4 m = *reinterpret_cast<const uint4*>(&sm.mask4[b][tid * kMaskCopies]);
      const uint32_t mb = (m.x | m.y) | (m.z | m.w);
      sm.mask[b][tid] = mb;
      u |= mb;
    }
    sm.umask[tid] = u;
    cnt = __popc(u);
  }
  const uint32_t inc = wave_scan_dpp(cnt);
  if (lane == kWave - 1) sm.wtot[w] = inc;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int ww = 0; ww < kNWB; ++ww) {
    before += ww < w ? sm.wtot[ww] : 0u;
    total += sm.wtot[ww];
  }
  if (tid < nw) sm.pre[tid] = before + inc - cnt;
  __syncthreads();
  const int n = int(total);   // rows of U in the range (uniform)
  if (tile == 0 && tid == 0) p.counts[split] = n;
  const bool col_ok = l16 * 8 < tile_w;
  const uint16_t* base;
  uint32_t stride;   // elements; the host keeps every row offset below 2^32
  if (p.tiled) {
    base = p.wt + size_t(tile) * kGemvTile * p.d_in + (col_ok ? l16 * 8 : 0);
    stride = uint32_t(tile_w);
  } else {
    base = p.wt + size_t(tile) * kGemvTile + (col_ok ? l16 * 8 : 0);
    stride = uint32_t(p.d_out);
  }
  // the ring reads up to 64 (nsteps + R - 1) positions: the padding past U's
  // rows re-reads the range's first row with input 0
  const int nsteps = (n + kSlotsB - 1) / kSlotsB;
  const int npad = kSlotsB * (nsteps + kRingB - 1);
  if (tid < npad - n) {
    sm.off[n + tid] = uint32_t(c0) * stride;
    sm.xf[n + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int r = kPerThread * tid + i;   // channel c0 + r
    if (c0 + r >= c1) continue;
    const int wd = r >> 5, bit = r & 31;
    const uint32_t u = sm.umask[wd];
    if (!((u >> bit) & 1u)) continue;
    const uint32_t pos = sm.pre[wd] + __popc(u & ((1u << bit) - 1u));
    float h[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NB; ++b) h[b] = ((sm.mask[b][wd] >> bit) & 1u) ? bf16_to_f32(uint16_t(xv[b][i])) : 0.f;
    sm.off[pos] = uint32_t(c0 + r) * stride;
    sm.xf[pos] = make_float4(h[0], h[1], h[2], h[3]);
  }
  __syncthreads();

  auto store = [&](int b, int c, float v) {
    if (p.n_splits == 1 && p.y)
      p.y[size_t(b) * p.d_out + tile * kGemvTile + c] = f32_to_bf16(v);
    else if (p.n_splits == 1)
      p.yf[size_t(b) * p.d_out + tile * kGemvTile + c] = v;
    else
      p.partial[(size_t(split) * NB + b) * p.d_out + tile * kGemvTile + c] = v;
  };
  if (n == 0) {   // no kept channel in the range
    for (int t = tid; t < NB * kGemvTile; t += kGemvThreads)
      if (t % kGemvTile < tile_w) store(t / kGemvTile, t % kGemvTile, 0.f);
    return;
  }

  auto load = [&](int j) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + sm.off[j]));
  };

  // ------------------------------------------------------------- row loop
  // as k_gemv's: a slot consumes its rows one at a time and refills each
  // right after, R rows ahead (4 rows in flight measured no faster at B = 4;
  // nor did pairing the two rows of a step for v_dot2)
  constexpr int R = kRingB;
  u32x4 ring[R];
#pragma unroll
  for (int u = 0; u < R; ++u) ring[u] = load(slot + kSlotsB * u);
  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = 0.f;
  auto consume = [&](int j, const u32x4& wv) {
    const float4 xr = sm.xf[j];
    const float xb[4] = {xr.x, xr.y, xr.z, xr.w};
    const float wf[8] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y),
                         bf16_lo(wv.z), bf16_hi(wv.z), bf16_lo(wv.w), bf16_hi(wv.w)};
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[b][c] += wf[c] * xb[b];
  };
  // every group of R steps but the last refills; the last only consumes
  int st = 0;
  for (; st + R < nsteps; st += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int j = slot + kSlotsB * (st + u);
      consume(j, ring[u]);
      ring[u] = load(j + R * kSlotsB);
    }
  }
#pragma unroll
  for (int u = 0; u < R; ++u) consume(slot + kSlotsB * (st + u), ring[u]);

  // ------------------------------------------------------------- epilogue
  // slot pairs (lanes l and l ^ 32) summed in registers, then the 32
  // half-wave sums through LDS in (wave, half) order: a second register step
  // would cost 8 B more cross-lane swaps per lane than the LDS reads it saves
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] += lane_xor<32>(acc[b][c]);
  if (lane < 32) {
    const int half = lane >> 4;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float4* rw = reinterpret_cast<float4*>(&sm.red[w][half][b][l16 * 8]);
      rw[0] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
      rw[1] = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
    }
  }
  __syncthreads();
  for (int t = tid; t < NB * kGemvTile; t += kGemvThreads) {
    const int b = t / kGemvTile, c = t % kGemvTile;
    if (c >= tile_w) continue;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNWB; ++ww) v += sm.red[ww][0][b][c] + sm.red[ww][1][b][c];
    store(b, c, v);
  }
}

// y[b][c] = bf16 of the sum of the range partials in range order
__global__ __launch_bounds__(256) void k_batch_finish(const BatchParams p) {
  const size_t n = size_t(p.nb) * p.d_out;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256) {
    float v = 0.f;
    for (int s = 0; s < p.n_splits; ++s) v += p.partial[size_t(s) * n + i];
    if (p.y)
      p.y[i] = f32_to_bf16(v);
    else
      p.yf[i] = v;
  }
}

// |U| = the sum of the ranges' row counts (only when the caller asks for it)
__global__ __launch_bounds__(256) void k_batch_count(const BatchParams p) {
  __shared__ int part[4];
  int v = 0;
  for (int s = threadIdx.x; s < p.n_splits; s += 256) v += p.counts[s];
  v = int(wave_sum_u32(uint32_t(v)));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) *p.count_out = part[0] + part[1] + part[2] + part[3];
}

template <int NB>
void launch_batch_nb(const BatchParams& p, dim3 grid, hipStream_t s) {
  k_gemv_batch<NB><<<grid, dim3(kGemvThreads), 0, s>>>(p);
}

}  // namespace
}  // namespace bc

using namespace bc;

extern "C" size_t bc_sparse_gemv_batch_workspace_bytes(int d_in, int d_out, int k, int batch) {
  if (d_in <= 0 || d_in > kBatchMaxIn || d_out <= 0 || k <= 0 || batch < 1 || batch > kBatchMax) return 0;
  return plan_batch(d_in, d_out, batch).bytes;
}

extern "C" int bc_sparse_gemv_batch(const uint16_t* wt, int tiled, int d_in, int d_out, const uint16_t* x,
                                    const int32_t* idx, int k, int batch, uint16_t* y, int32_t* n_union_out,
                                    void* ws, size_t ws_bytes, void* stream) {
  const char* name = "bc_sparse_gemv_batch";
  if (!wt || !x || !y) return set_error(BC_ERR_INVALID, "%s: NULL pointer", name);
  if (batch < 1 || batch > kBatchMax)
    return set_error(BC_ERR_UNSUPPORTED, "%s: batch %d outside [1, %d]", name, batch, kBatchMax);
  if (d_in <= 0 || d_out <= 0) return set_error(BC_ERR_INVALID, "%s: d_in=%d d_out=%d", name, d_in, d_out);
  if (d_in > kBatchMaxIn) return set_error(BC_ERR_UNSUPPORTED, "%s: d_in %d > %d", name, d_in, kBatchMaxIn);
  if (d_out % 8 != 0) return set_error(BC_ERR_UNSUPPORTED, "%s: d_out %% 8 != 0 (%d)", name, d_out);
  if (idx == nullptr) {
    if (k != d_in) return set_error(BC_ERR_INVALID, "%s: dense call needs k == d_in", name);
  } else if (k < 1 || k > d_in) {
    return set_error(BC_ERR_INVALID, "%s: k=%d outside [1, %d]", name, k, d_in);
  }
  if ((reinterpret_cast<uintptr_t>(wt) | reinterpret_cast<uintptr_t>(ws)) & 15)
    return set_error(BC_ERR_INVALID, "%s: wt and ws must be 16-byte aligned", name);
  if (!tiled && size_t(d_in) * size_t(d_out) > 0xFFFFFFFFull)
    return set_error(BC_ERR_UNSUPPORTED, "%s: row-major W^T of %d x %d (use the tiled layout)", name, d_in, d_out);
  return run_gemv_batch(wt, tiled, d_in, d_out, x, idx, k, batch, y, nullptr, n_union_out, ws, ws_bytes,
                        static_cast<hipStream_t>(stream));
}

int bc::run_gemv_batch(const uint16_t* wt, int tiled, int d_in, int d_out, const uint16_t* x, const int32_t* idx,
                       int k, int batch, uint16_t* y, float* yf, int32_t* n_union_out, void* ws, size_t ws_bytes,
                       hipStream_t s) {
  const char* name = "batched GEMV";
  const BatchPlan pl = plan_batch(d_in, d_out, batch);
  if (!ws || ws_bytes < pl.bytes)
    return set_error(BC_ERR_WORKSPACE, "%s: workspace %zu < %zu", name, ws_bytes, pl.bytes);
  char* w = static_cast<char*>(ws);
  BatchParams p{};
  p.wt = wt; p.tiled = tiled ? 1 : 0; p.d_in = d_in; p.d_out = d_out; p.k = k; p.nb = batch;
  p.x = x; p.idx = idx; p.range = pl.range; p.n_splits = pl.n_splits;
  p.counts = reinterpret_cast<int32_t*>(w);
  p.count_out = n_union_out;
  p.partial = pl.n_splits > 1 ? reinterpret_cast<float*>(w + pl.off_part) : nullptr;
  p.y = y;
  p.yf = yf;
  const dim3 grid(pl.n_tiles, pl.n_splits);
  switch (batch) {
    case 1: launch_batch_nb<1>(p, grid, s); break;
    case 2: launch_batch_nb<2>(p, grid, s); break;
    case 3: launch_batch_nb<3>(p, grid, s); break;
    default: launch_batch_nb<4>(p, grid, s); break;
  }
  int rc = check_launch("k_gemv_batch");
  if (rc != BC_OK) return rc;
  if (pl.n_splits > 1) {
    const size_t total = size_t(batch) * d_out;
    const int groups = total / 256 + 1 < 1024 ? int(total / 256 + 1) : 1024;
    k_batch_finish<<<groups, 256, 0, s>>>(p);
    if ((rc = check_launch("k_batch_finish")) != BC_OK) return rc;
  }
  if (n_union_out) {
    k_batch_count<<<1, 256, 0, s>>>(p);
    rc = check_launch("k_batch_count");
  }
  return rc;
}
