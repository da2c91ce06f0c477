// Preparation kernels:
//  * ln_in: the LayerNorm applied to x before f1 (page "4.4 Scaling
//    Recommendation Models", section "Code": norm_in ahead of f1), one wave per
//    row held in registers, fp32 statistics, biased variance.
//  * build_tiles: the attention work list for jagged batches — one item per
//    (sequence, 128-row query tile), ordered by decreasing work so the longest
//    items start first (kernels that skip the padding of variable-length
//    sequences: "Efficiency tricks" paragraph of the same page), plus the
//    list of all 64-key blocks;
//  * block_ts: per 64-key block, the earliest and latest timestamp and each
//    key's offset from the earliest — head- and query-independent facts that
//    every attention workgroup streaming the block would otherwise recompute.
#include "common.h"
#include "kernels.h"

namespace hstu {

// The row stays in registers between the statistics and the output: NC
// 16-byte chunks per lane cover rows of up to NC * 64 * V elements, so x is
// read from HBM once.
template <typename T, int NC>
__global__ __launch_bounds__(256) void ln_in_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                    const T* __restrict__ b, T* __restrict__ y,
                                                    int64_t rows, int d, float eps) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= rows) return;  // whole wave leaves together
  const T* xr = x + row * d;
  T* yr = y + row * d;
  uint4 xv[NC];
  float f[V], gg[V], bb[V];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = (k * kWave + lane) * V;
    if (c < d) {
      xv[k] = ld16(xr + c);
      unpack(xv[k], f, T());
#pragma unroll
      for (int e = 0; e < V; ++e) s += f[e];
    }
  }
  const float mean = wave_sum(s) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    if ((k * kWave + lane) * V < d) {
      unpack(xv[k], f, T());
#pragma unroll
      for (int e = 0; e < V; ++e) q += (f[e] - mean) * (f[e] - mean);
    }
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)d + eps);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = (k * kWave + lane) * V;
    if (c < d) {
      unpack(xv[k], f, T());
      unpack(ld16(g + c), gg, T());
      unpack(ld16(b + c), bb, T());
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = (f[e] - mean) * rstd * gg[e] + bb[e];
      st16(yr + c, pack(f, T()));
    }
  }
}

template <typename T>
static hipError_t launch_ln_in_t(const void* x, const void* g, const void* b, void* y, int64_t T_,
                                 int d, float eps, hipStream_t s) {
  const dim3 grid((unsigned)((T_ + 3) / 4)), block(256);
  const int per_lane = (d / Elem<T>::kVec + kWave - 1) / kWave;  // chunks per lane
#define HSTU_LN_CASE(NC)                                                                           \
  if (per_lane <= NC) {                                                                            \
    hipLaunchKernelGGL((ln_in_kernel<T, NC>), grid, block, 0, s, (const T*)x, (const T*)g, (const T*)b, \
                       (T*)y, T_, d, eps);                                                         \
    return hipGetLastError();                                                                      \
  }
  HSTU_LN_CASE(1)
  HSTU_LN_CASE(2)
  HSTU_LN_CASE(4)
  HSTU_LN_CASE(8)
  HSTU_LN_CASE(16)
  HSTU_LN_CASE(32)
#undef HSTU_LN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_ln_in(hstu_dtype dt, const void* x, const void* g, const void* b, void* y,
                        int64_t T, int d, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dt == HSTU_BF16) return launch_ln_in_t<bf16>(x, g, b, y, T, d, eps, s);
  return launch_ln_in_t<float>(x, g, b, y, T, d, eps, s);
}

// ------------------------------------------------------------ work list
constexpr int kCostBuckets = 2048;
constexpr int kTileThreads = 1024;

// Keys a work item touches: the history keys up to its tile's last row, plus
// one key block for the candidates' own diagonal; in a cached pass (klen >= 0)
// the key blocks of its history chunk.
__device__ __forceinline__ int tile_cost_bucket(const SeqInfo& si, int qt, int bm, int klen, int ns, int c) {
  int i0 = qt * bm;
  int iend = min(i0 + bm, si.len);
  int cost;
  if (klen >= 0) {
    int lo, hi;
    cand_chunk((klen + kAttnBN - 1) / kAttnBN, ns, c, lo, hi);
    cost = (hi - lo) * kAttnBN;
  } else {
    cost = min(iend, si.nhist) + (iend > si.nhist ? kAttnBN : 0);
  }
  return min(kCostBuckets - 1, cost >> 4);
}

// Exclusive prefix sum of v over the workgroup's kTileThreads threads; the
// sum of all v goes to total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* part, int& total) {
  const int tid = threadIdx.x;
  part[tid] = v;
  __syncthreads();
  for (int o = 1; o < kTileThreads; o <<= 1) {
    const int u = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += u;
    __syncthreads();
  }
  const int incl = part[tid];
  total = part[kTileThreads - 1];
  __syncthreads();
  return incl - v;
}

// Largest b in [0, B) with base[b] <= g: the sequence whose items
// [base[b], base[b + 1]) hold item g (empty sequences are skipped).
__device__ __forceinline__ int owner(const int32_t* base, int B, int g) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= g)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// One workgroup.  Items are spread over the threads through per-sequence
// prefix sums (tbase, kbase: first tile / key block of each sequence), so the
// work does not serialise on a few long sequences.  Tiles cover the query
// rows (off, ncand, T); key blocks cover the key rows (koff, Tk), which are
// the same rows unless the pass reads a cached history.
__global__ __launch_bounds__(kTileThreads) void build_tiles_kernel(const int64_t* __restrict__ off,
                                                                   const int32_t* __restrict__ ncand,
                                                                   int32_t B, int64_t T, int bm,
                                                                   const int64_t* __restrict__ koff,
                                                                   int64_t Tk, int cached,
                                                                   int64_t max_tiles,
                                                                   int2* __restrict__ tiles,
                                                                   int64_t max_kblocks,
                                                                   int2* __restrict__ kblocks,
                                                                   int32_t* __restrict__ tbase,
                                                                   int32_t* __restrict__ kbase,
                                                                   int32_t* __restrict__ nsplit,
                                                                   int32_t* __restrict__ count) {
  __shared__ int hist[kCostBuckets];
  __shared__ int part[kTileThreads];
  const int tid = threadIdx.x;
  for (int i = tid; i < kCostBuckets; i += kTileThreads) hist[i] = 0;
  auto klen = [&](int b) { return cached ? seq_info(koff, nullptr, b, Tk).len : -1; };
  auto splits = [&](int b) { return cached ? cand_nsplit(klen(b)) : 1; };

  // Per-sequence item counts -> exclusive bases.
  int run_t = 0, run_k = 0;
  for (int b0 = 0; b0 < B; b0 += kTileThreads) {
    const int b = b0 + tid;
    int nt = 0, nk = 0;
    if (b < B) {
      const SeqInfo si = seq_info(off, ncand, b, T);
      const int ns = splits(b);
      nt = (si.len + bm - 1) / bm * ns;
      nk = ((cached ? klen(b) : si.len) + kAttnBN - 1) / kAttnBN;
      nsplit[b] = ns;
    }
    int tot_t, tot_k;
    const int et = block_exclusive_scan(nt, part, tot_t);
    const int ek = block_exclusive_scan(nk, part, tot_k);
    if (b < B) {
      tbase[b] = run_t + et;
      kbase[b] = run_k + ek;
    }
    run_t += tot_t;
    run_k += tot_k;
  }
  const int total = (int)min((int64_t)run_t, max_tiles), total_k = (int)min((int64_t)run_k, max_kblocks);
  __syncthreads();

  // Histogram of tile costs; the key-block list in sequence order.
  // item k of sequence b: query tile k / ns, history chunk k % ns
  for (int g = tid; g < total; g += kTileThreads) {
    const int b = owner(tbase, B, g), ns = splits(b), k = g - tbase[b];
    atomicAdd(&hist[tile_cost_bucket(seq_info(off, ncand, b, T), k / ns, bm, klen(b), ns, k % ns)], 1);
  }
  for (int g = tid; g < total_k; g += kTileThreads) {
    const int b = owner(kbase, B, g);
    kblocks[g] = make_int2(b, g - kbase[b]);
  }
  __syncthreads();
  // Exclusive scan in decreasing-cost order: start[k] = sum of hist[k'] for k' > k.
  // Thread t owns the two buckets 2047-2t and 2046-2t.
  const int hi = kCostBuckets - 1 - 2 * tid, lo = hi - 1;
  const int h_hi = hist[hi], h_lo = hist[lo];
  int dummy;
  const int before = block_exclusive_scan(h_hi + h_lo, part, dummy);
  hist[hi] = before;
  hist[lo] = before + h_hi;
  __syncthreads();
  for (int g = tid; g < total; g += kTileThreads) {
    const int b = owner(tbase, B, g), ns = splits(b), k = g - tbase[b];
    const int qt = k / ns, c = k % ns;
    const int pos = atomicAdd(&hist[tile_cost_bucket(seq_info(off, ncand, b, T), qt, bm, klen(b), ns, c)], 1);
    tiles[pos] = make_int2(b, qt | (c << 24));
  }
  if (tid == 0) {
    count[0] = total;
    count[1] = total_k;
  }
}

// One wave per key block: min / max of its timestamps and each key's offset
// from the min (meaningful when the block spans at most INT32_MAX; the
// attention kernel checks that from tstat before using rel); with token types
// (nt > 0) each key's type, clamped to nt - 1, as int32.
__global__ __launch_bounds__(256) void block_ts_kernel(const int64_t* __restrict__ off,
                                                       const int32_t* __restrict__ ncand, int64_t T,
                                                       const int64_t* __restrict__ ts,
                                                       const int2* __restrict__ kblocks,
                                                       const int32_t* __restrict__ count,
                                                       int32_t* __restrict__ rel,
                                                       int64_t* __restrict__ tstat,
                                                       const uint8_t* __restrict__ types, int nt,
                                                       int32_t* __restrict__ kty) {
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
  if (valid && nt > 0) kty[si.start + j] = min((int)types[si.start + j], nt - 1);
  if (lane == 0) {
    tstat[2 * (si.start + e.y * kAttnBN)] = mn;
    tstat[2 * (si.start + e.y * kAttnBN) + 1] = mx;
  }
}

hipError_t launch_attn_prep(const AttnRows& r, int bm, const AttnScratch& sc, hipStream_t s) {
  const int64_t max_kb = attn_max_kblocks(r.Tk, r.B);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kTileThreads), 0, s, r.qoff, r.ncand, r.B, r.Tq, bm, r.koff,
                     r.Tk, r.cached ? 1 : 0, attn_max_items(r.Tq, r.B, r.cached), sc.tiles, max_kb, sc.kblocks,
                     sc.tbase, sc.kbase, sc.nsplit, sc.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_ts_kernel, dim3((unsigned)((max_kb + 3) / 4)), dim3(256), 0, s, r.koff,
                     (const int32_t*)nullptr, r.Tk, r.kts, sc.kblocks, sc.counts, sc.rel, sc.tstat, r.types.k,
                     r.types.nt, sc.kty);
  return hipGetLastError();
}

}  // namespace hstu
