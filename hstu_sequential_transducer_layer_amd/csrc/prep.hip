// Preparation kernels:
//  * ln_in: the LayerNorm applied to x before f1 (page "4.4 Scaling
//    Recommendation Models", section "Code": norm_in ahead of f1), one wave per
//    row, fp32 statistics, biased variance.
//  * build_tiles: the attention work list for jagged batches — one item per
//    (sequence, 128-row query tile), ordered by decreasing work so the longest
//    items start first (the pages' "sparsity-aware kernels for variable-length
//    sequences", "Efficiency tricks" paragraph of the same page).
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
__device__ __forceinline__ int tile_cost_bucket(const SeqInfo& si, int qt) {
  int i0 = qt * kAttnBM;
  int iend = min(i0 + kAttnBM, si.len);
  int cost = min(iend, si.nhist) + (iend > si.nhist ? kAttnBN : 0);
  return min(kCostBuckets - 1, cost >> 4);
}

__global__ __launch_bounds__(kTileThreads) void build_tiles_kernel(const int64_t* __restrict__ off,
                                                                   const int32_t* __restrict__ ncand,
                                                                   int32_t B, int64_t T,
                                                                   int64_t max_tiles,
                                                                   int2* __restrict__ tiles,
                                                                   int32_t* __restrict__ count) {
  __shared__ int hist[kCostBuckets];
  __shared__ int part[kTileThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < kCostBuckets; i += kTileThreads) hist[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kTileThreads) {
    SeqInfo si = seq_info(off, ncand, b, T);
    int nt = (si.len + kAttnBM - 1) / kAttnBM;
    for (int qt = 0; qt < nt; ++qt) atomicAdd(&hist[tile_cost_bucket(si, qt)], 1);
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
    int nt = (si.len + kAttnBM - 1) / kAttnBM;
    for (int qt = 0; qt < nt; ++qt) {
      int pos = atomicAdd(&hist[tile_cost_bucket(si, qt)], 1);
      if (pos < max_tiles) tiles[pos] = make_int2(b, qt);
    }
  }
  if (tid == 0) *count = (int32_t)min((int64_t)total, max_tiles);
}

hipError_t launch_build_tiles(const int64_t* off, const int32_t* ncand, int32_t B, int64_t T,
                              int2* tiles, int32_t* tiles_count, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, off, ncand, B, T,
                     attn_max_tiles(T, B), tiles, tiles_count);
  return hipGetLastError();
}

}  // namespace hstu
