// Stochastic length on the device — page "HSTU: The First Exploration of the
// Scaling Law", 7.1.5 Engineering Optimizations, "Stochastic Length": a
// sequence of n tokens longer than N^(alpha/2) is, with probability
// 1 - N^alpha / n^2, replaced by floor(N^(alpha/2)) of its tokens.  The random
// draws are inputs (one uniform per sequence, one uint32 key per token); the
// subsequence is the k tokens with the smallest (key, position), kept in
// position order.  Three kernels: the plan (decisions and new offsets, one
// workgroup), the selection (one workgroup per sequence: radix select of the
// k-th smallest key in four 8-bit passes, then an order-preserving compaction)
// and a row gather that re-packs any per-row tensor.
#include "common.h"
#include "kernels.h"

namespace hstu {

constexpr int kSlThreads = 256;

// Exclusive scan over the workgroup's 256 threads; `total` gets the sum.
// part: 4 ints of LDS.  Every thread must call it.
__device__ __forceinline__ int sl_block_scan(int v, int* part, int& total) {
  const int lane = threadIdx.x & 63, w = wave_id();
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) part[w] = x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kSlThreads / kWave; ++i) before += i < w ? part[i] : 0;
  total = part[0] + part[1] + part[2] + part[3];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kSlThreads) void sl_plan_kernel(const int64_t* __restrict__ off, int32_t B, int64_t T,
                                                             const float* __restrict__ u, double thr, int64_t k,
                                                             double na, int64_t* __restrict__ new_off,
                                                             int32_t* __restrict__ trunc) {
  __shared__ int part[kSlThreads / kWave];
  const int tid = threadIdx.x;
  int64_t run = 0;
  for (int b0 = 0; b0 < B; b0 += kSlThreads) {
    const int b = b0 + tid;
    int kept = 0;
    if (b < B) {
      const SeqInfo si = seq_info(off, nullptr, b, T);
      const double n = (double)si.len;
      const bool t = n > thr && (double)u[b] < 1.0 - na / (n * n);
      kept = t ? (int)k : si.len;
      trunc[b] = t ? 1 : 0;
    }
    int tot;
    const int ex = sl_block_scan(kept, part, tot);
    if (b < B) new_off[b] = run + ex;
    run += tot;
  }
  if (tid == 0) new_off[B] = run;
}

__global__ __launch_bounds__(kSlThreads) void sl_select_kernel(const int64_t* __restrict__ off, int32_t B, int64_t T,
                                                               const uint32_t* __restrict__ keys, int64_t k,
                                                               const int64_t* __restrict__ new_off,
                                                               const int32_t* __restrict__ trunc,
                                                               int64_t* rows) {
  __shared__ int hist[256];
  __shared__ int part[kSlThreads / kWave];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem;
  const int tid = threadIdx.x, b = blockIdx.x;
  const SeqInfo si = seq_info(off, nullptr, b, T);
  const int n = si.len;
  const int64_t s0 = si.start;
  // rows has T entries; with well-formed offsets every write lands below T,
  // and the bound keeps malformed ones (clamped by seq_info) inside it
  const int64_t base = new_off[b];
  auto put = [&](int64_t at, int64_t v) {
    if (base + at >= 0 && base + at < T) rows[base + at] = v;
  };
  if (!trunc[b]) {
    for (int i = tid; i < n; i += kSlThreads) put(i, s0 + i);
    return;
  }
  // The k-th smallest key K* (k counted from 1), 8 bits at a time from the top;
  // rem ends as the number of keys equal to K* that are kept.
  uint32_t prefix = 0, mask = 0;
  int rem = (int)min<int64_t>(k, n);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSlThreads) {
      const uint32_t key = keys[s0 + i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int c = 0, d = 0;
      for (; d < 255; ++d) {
        if (c + hist[d] >= rem) break;
        c += hist[d];
      }
      sh_prefix = prefix | ((uint32_t)d << shift);
      sh_rem = rem - c;
    }
    __syncthreads();
    prefix = sh_prefix;
    rem = sh_rem;
    mask |= 255u << shift;
  }
  // Keep keys below K* and the first rem keys equal to it, in position order.
  int taken_eq = 0, out = 0;
  for (int c0 = 0; c0 < n; c0 += kSlThreads) {
    const int i = c0 + tid;
    const uint32_t key = i < n ? keys[s0 + i] : 0u;
    const bool lt = i < n && key < prefix, eq = i < n && key == prefix;
    int tot_eq, tot_keep;
    const int rank_eq = sl_block_scan(eq ? 1 : 0, part, tot_eq);
    const bool keep = lt || (eq && taken_eq + rank_eq < rem);
    const int pos = sl_block_scan(keep ? 1 : 0, part, tot_keep);
    if (keep) put(out + pos, s0 + i);
    taken_eq += tot_eq;
    out += tot_keep;
  }
}

hipError_t launch_sl_sample(const int64_t* off, int32_t B, int64_t T, const float* u, const uint32_t* keys,
                            double thr, int64_t k, double na, int64_t* new_off, int64_t* rows, int32_t* trunc,
                            hipStream_t s) {
  hipLaunchKernelGGL(sl_plan_kernel, dim3(1), dim3(kSlThreads), 0, s, off, B, T, u, thr, k, na, new_off, trunc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || B == 0) return e;
  hipLaunchKernelGGL(sl_select_kernel, dim3((unsigned)B), dim3(kSlThreads), 0, s, off, B, T, keys, k, new_off,
                     trunc, rows);
  return hipGetLastError();
}

// dst row r = src row rows[r] for r < min(*count, max_rows); W-byte words.
template <typename W>
__global__ __launch_bounds__(256) void gather_rows_kernel(const W* __restrict__ src, int64_t src_rows,
                                                          int64_t words, const int64_t* __restrict__ rows,
                                                          const int64_t* __restrict__ count, int64_t max_rows,
                                                          W* __restrict__ dst) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = t / words, c = t - r * words;
  const int64_t n = min(max(*count, (int64_t)0), max_rows);
  if (r >= n) return;
  const int64_t sr = min(max(rows[r], (int64_t)0), src_rows - 1);
  dst[r * words + c] = src[sr * words + c];
}

hipError_t launch_gather_rows(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* rows,
                              const int64_t* count, int64_t max_rows, void* dst, hipStream_t s) {
  if (max_rows == 0 || src_rows == 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t al = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
#define HSTU_GATHER(W_)                                                                                  \
  {                                                                                                     \
    const int64_t words = row_bytes / (int64_t)sizeof(W_);                                              \
    const int64_t grid = (max_rows * words + 255) / 256;                                                \
    hipLaunchKernelGGL(gather_rows_kernel<W_>, dim3((unsigned)grid), dim3(256), 0, s, (const W_*)src,    \
                       src_rows, words, rows, count, max_rows, (W_*)dst);                               \
    return hipGetLastError();                                                                          \
  }
  if (al % 16 == 0) HSTU_GATHER(uint4)
  if (al % 8 == 0) HSTU_GATHER(uint2)
  if (al % 4 == 0) HSTU_GATHER(uint32_t)
  HSTU_GATHER(uint8_t)
#undef HSTU_GATHER
}

}  // namespace hstu
