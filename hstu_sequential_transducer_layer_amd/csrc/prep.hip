// Preparation kernels:
//  * ln_in: the LayerNorm applied to x before f1 (page "4.4 Scaling
//    Recommendation Models", section "Code": norm_in ahead of f1), one wave per
//    row, fp32 statistics, biased variance.
//  * build_tiles: the attention work list for jagged batches — one item per
//    (sequence, 128-row query tile), ordered by decreasing work so the longest
//    items start first (the pages' "sparsity-aware kernels for variable-length
//    sequences", "Efficiency tricks" paragraph of the same page), plus the
//    list of all 64-key blocks;
//  * block_ts: per 64-key block, the earliest and latest timestamp and each
//    key's offset from the earliest — head- and query-independent facts that
//    every attention workgroup streaming the block would otherwise recompute.
#include "common.h"
#include "kernels.h"

namespace hstu {

template <typename T>
__global__ __launch_bounds__(256) void ln_in_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                    const T* __restrict__ b, T* __restrict__ y,
                                                    int64_t rows, int d, float eps) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= rows) return;  // whole wave leaves together
  const T* xr = x + row * d;
  T* yr = y + row * d;
  float f[V], gg[V], bb[V];
  float s = 0.f;
  for (int c = lane * V; c < d; c += kWave * V) {
    unpack(ld16(xr + c), f, T());
#pragma unroll
    for (int e = 0; e < V; ++e) s += f[e];
  }
  const float mean = wave_sum(s) / (float)d;
  float q = 0.f;
  for (int c = lane * V; c < d; c += kWave * V) {
    unpack(ld16(xr + c), f, T());
#pragma unroll
    for (int e = 0; e < V; ++e) q += (f[e] - mean) * (f[e] - mean);
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)d + eps);
  for (int c = lane * V; c < d; c += kWave * V) {
    unpack(ld16(xr + c), f, T());
    unpack(ld16(g + c), gg, T());
    unpack(ld16(b + c), bb, T());
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = (f[e] - mean) * rstd * gg[e] + bb[e];
    st16(yr + c, pack(f, T()));
  }
}

hipError_t launch_ln_in(hstu_dtype dt, const void* x, const void* g, const void* b, void* y,
                        int64_t T, int d, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (dt == HSTU_BF16)
    hipLaunchKernelGGL(ln_in_kernel<bf16>, grid, block, 0, s, (const bf16*)x, (const bf16*)g,
                       (const bf16*)b, (bf16*)y, T, d, eps);
  else
    hipLaunchKernelGGL(ln_in_kernel<float>, grid, block, 0, s, (const float*)x, (const float*)g,
                       (const float*)b, (float*)y, T, d, eps);
  return hipGetLastError();
}

// ------------------------------------------------------------ work list
constexpr int kCostBuckets = 2048;
constexpr int kTileThreads = 1024;

// Keys a query tile touches: the history keys up to its last row, plus one
// key block for the candidates' own diagonal.
__device__ __forceinline__ int tile_cost_bucket(const SeqInfo& si, int qt, int bm) {
  int i0 = qt * bm;
  int iend = min(i0 + bm, si.len);
  int cost = min(iend, si.nhist) + (iend > si.nhist ? kAttnBN : 0);
  return min(kCostBuckets - 1, cost >> 4);
}

__global__ __launch_bounds__(kTileThreads) void build_tiles_kernel(const int64_t* __restrict__ off,
                                                                   const int32_t* __restrict__ ncand,
                                                                   int32_t B, int64_t T, int bm,
                                                                   int64_t max_tiles,
                                                                   int2* __restrict__ tiles,
                                                                   int64_t max_kblocks,
                                                                   int2* __restrict__ kblocks,
                                                                   int32_t* __restrict__ count) {
  __shared__ int hist[kCostBuckets];
  __shared__ int part[kTileThreads];
  __shared__ int nkb;
  const int tid = threadIdx.x;
  for (int i = tid; i < kCostBuckets; i += kTileThreads) hist[i] = 0;
  if (tid == 0) nkb = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kTileThreads) {
    SeqInfo si = seq_info(off, ncand, b, T);
    int nt = (si.len + bm - 1) / bm;
    for (int qt = 0; qt < nt; ++qt) atomicAdd(&hist[tile_cost_bucket(si, qt, bm)], 1);
  }
  __syncthreads();
  // Exclusive scan in decreasing-cost order: start[k] = sum of hist[k'] for k' > k.
  // Thread t owns the two buckets 2047-2t and 2046-2t.
  const int hi = kCostBuckets - 1 - 2 * tid, lo = hi - 1;
  const int h_hi = hist[hi], h_lo = hist[lo];
  part[tid] = h_hi + h_lo;
  __syncthreads();
  for (int o = 1; o < kTileThreads; o <<= 1) {
    int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int before = part[tid] - (h_hi + h_lo);
  const int total = part[kTileThreads - 1];
  __syncthreads();
  hist[hi] = before;
  hist[lo] = before + h_hi;
  __syncthreads();
  for (int b = tid; b < B; b += kTileThreads) {
    SeqInfo si = seq_info(off, ncand, b, T);
    int nt = (si.len + bm - 1) / bm;
    for (int qt = 0; qt < nt; ++qt) {
      int pos = atomicAdd(&hist[tile_cost_bucket(si, qt, bm)], 1);
      if (pos < max_tiles) tiles[pos] = make_int2(b, qt);
    }
    const int nb = (si.len + kAttnBN - 1) / kAttnBN;
    const int kpos = nb > 0 ? atomicAdd(&nkb, nb) : 0;
    for (int kb = 0; kb < nb; ++kb)
      if (kpos + kb < max_kblocks) kblocks[kpos + kb] = make_int2(b, kb);
  }
  __syncthreads();
  if (tid == 0) {
    count[0] = (int32_t)min((int64_t)total, max_tiles);
    count[1] = (int32_t)min((int64_t)nkb, max_kblocks);
  }
}

// One wave per key block: min / max of its timestamps and each key's offset
// from the min (meaningful when the block spans at most INT32_MAX; the
// attention kernel checks that from tstat before using rel).
__global__ __launch_bounds__(256) void block_ts_kernel(const int64_t* __restrict__ off,
                                                       const int32_t* __restrict__ ncand, int64_t T,
                                                       const int64_t* __restrict__ ts,
                                                       const int2* __restrict__ kblocks,
                                                       const int32_t* __restrict__ count,
                                                       int32_t* __restrict__ rel,
                                                       int64_t* __restrict__ tstat) {
  const int lane = threadIdx.x & 63;
  const int64_t id = (int64_t)blockIdx.x * 4 + wave_id();
  if (id >= count[1]) return;  // whole wave leaves together
  const int2 e = kblocks[id];
  const SeqInfo si = seq_info(off, ncand, e.x, T);
  const int j = e.y * kAttnBN + lane;
  const bool valid = j < si.len;
  const int64_t t = valid ? ts[si.start + j] : 0;
  int64_t mn = valid ? t : INT64_MAX, mx = valid ? t : INT64_MIN;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t omn = __shfl_xor(mn, o, kWave), omx = __shfl_xor(mx, o, kWave);
    mn = omn < mn ? omn : mn;
    mx = omx > mx ? omx : mx;
  }
  if (valid) rel[si.start + j] = (int32_t)(uint32_t)((uint64_t)t - (uint64_t)mn);
  if (lane == 0) {
    tstat[2 * (si.start + e.y * kAttnBN)] = mn;
    tstat[2 * (si.start + e.y * kAttnBN) + 1] = mx;
  }
}

hipError_t launch_attn_prep(const int64_t* off, const int32_t* ncand, int32_t B, int64_t T,
                            const int64_t* ts, int bm, const AttnScratch& sc, hipStream_t s) {
  const int64_t max_kb = attn_max_kblocks(T, B);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, off, ncand, B, T, bm,
                     attn_max_tiles(T, B), sc.tiles, max_kb, sc.kblocks, sc.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_ts_kernel, dim3((unsigned)((max_kb + 3) / 4)), dim3(256), 0, s, off, ncand, T, ts,
                     sc.kblocks, sc.counts, sc.rel, sc.tstat);
  return hipGetLastError();
}

}  // namespace hstu
