// Inspection entry point: the integer indexing of the attention stage for
// arbitrary (query row, key row) pairs, computed with the same device
// functions the attention kernel uses (row -> sequence by binary search over
// the clamped offsets; positions with the shared candidate slot; relative
// position bucket; log time bucket; causal + candidate mask).  Definitions:
// page "4.4 Scaling Recommendation Models", section "Generative Recommenders
// and HSTU" (bias on position and time difference, candidate mask) and page
// "HSTU: The First Exploration of the Scaling Law", 7.1.4 Innovation 2.
#include "common.h"
#include "kernels.h"

namespace hstu {

__device__ int find_seq(const int64_t* off, const int32_t* ncand, int B, int64_t T, int64_t row) {
  // last b with start(b) <= row < start(b) + len(b), scanning clamped offsets
  int lo = 0, hi = B - 1, ans = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const SeqInfo si = seq_info(off, ncand, mid, T);
    if (si.start <= row) {
      ans = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  // skip back over empty sequences that start at the same row
  while (ans >= 0) {
    const SeqInfo si = seq_info(off, ncand, ans, T);
    if (row < si.start + si.len) return ans;
    if (si.len > 0) return -1;
    --ans;
  }
  return -1;
}

__global__ void debug_indices_kernel(const int64_t* __restrict__ off, const int32_t* __restrict__ ncand,
                                     int B, int64_t T, const int64_t* __restrict__ ts,
                                     const int64_t* __restrict__ pairs, int64_t n,
                                     int64_t* __restrict__ out, int P, int NB, int sbits, int shared) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int64_t qr = pairs[2 * t], kr = pairs[2 * t + 1];
  int64_t* o = out + 6 * t;
  for (int e = 0; e < 6; ++e) o[e] = 0;
  o[0] = -1;
  if (qr < 0 || qr >= T || kr < 0 || kr >= T) return;
  const int bq = find_seq(off, ncand, B, T, qr);
  if (bq < 0) return;
  const SeqInfo si = seq_info(off, ncand, bq, T);
  if (kr < si.start || kr >= si.start + si.len) return;
  const int i = (int)(qr - si.start), j = (int)(kr - si.start);
  const int R = (P - 1) / 2;
  o[0] = bq;
  o[1] = i;
  o[2] = j;
  o[3] = pos_bucket(position(i, si.nhist, shared != 0), position(j, si.nhist, shared != 0), R);
  o[4] = time_bucket(wrap_sub(ts[qr], ts[kr]), NB, sbits);
  o[5] = attends(i, j, si.nhist) ? 1 : 0;
}

hipError_t launch_debug_indices(const hstu_desc& d, const int64_t* off, const int32_t* ncand,
                                int32_t B, int64_t T, const int64_t* ts, const int64_t* pairs,
                                int64_t n, int64_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blk = 256;
  hipLaunchKernelGGL(debug_indices_kernel, dim3((unsigned)((n + blk - 1) / blk)), dim3(blk), 0, s,
                     off, ncand, B, T, ts, pairs, n, out, d.pos_buckets, d.time_buckets,
                     d.time_sub_bits, (d.flags & HSTU_CAND_SHARED_POS) ? 1 : 0);
  return hipGetLastError();
}

}  // namespace hstu
