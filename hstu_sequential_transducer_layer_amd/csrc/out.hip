// Stage 3: Y = f2(LayerNorm(AV) * U) + b2 (+ x) — page "4.4 Scaling
// Recommendation Models", section "Generative Recommenders and HSTU" (third
// layer equation; gating in place of an FFN) and section "Code" (LayerNorm over
// the merged heads, multiply by u, f2, residual add); page "HSTU: The First
// Exploration of the Scaling Law", 7.1.4 Innovation 1 (LayerNorm(AV) * U).
//
// Two kernels:
//  * gate: Z = (LayerNorm(AV) * g + b) * U, one wave per row, reading the
//    per-head-centred AV, the fp32 per-(row, head) statistics written by the
//    attention kernel and U once each (HBM-bound).  Row statistics are merged
//    from the H head partials with the parallel-variance formula:
//    mean = avg_h mean_h, M2 = sum_h M2_h + dv * sum_h (mean_h - mean)^2, so no
//    bf16-rounded value ever enters a variance.
//  * f2: the MFMA GEMM Z W2^T with + b2 and the residual in its epilogue.
// Producing Z inside the GEMM's operand load instead would redo the gate once
// per output-column tile (d_model / 256 times) and hold its inputs in
// registers next to the accumulators; writing Z once and reading it back costs
// one extra pass over T x H*dv elements.
#include "common.h"
#include "gemm.h"
#include "gemm2.h"
#include "kernels.h"

namespace hstu {

// One wave per row; K = H * dv columns, head h owning [h*dv, (h+1)*dv).
template <typename T>
__global__ __launch_bounds__(256) void gate_kernel(const T* __restrict__ av, const T* __restrict__ u,
                                                   const float* __restrict__ stats,
                                                   const T* __restrict__ g, const T* __restrict__ be,
                                                   T* __restrict__ z, int64_t M, int H, int dv,
                                                   float eps) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= M) return;  // whole wave leaves together
  const int K = H * dv;
  // lane h < H holds head h's partials
  const float2 st = lane < H ? reinterpret_cast<const float2*>(stats)[row * H + lane] : make_float2(0.f, 0.f);
  const float mean = wave_sum(st.x) / (float)H;
  const float dm = st.x - mean;
  const float m2 = wave_sum(lane < H ? st.y + (float)dv * dm * dm : 0.f);
  const float rstd = rsqrtf(m2 / (float)K + eps);
  const T* ar = av + row * K;
  const T* ur = u + row * K;
  T* zr = z + row * K;
#pragma unroll 2
  for (int c = lane * V; c < K; c += kWave * V) {
    float a[V], uu[V], gg[V], bb[V], o[V];
    unpack(ld16(ar + c), a, T());
    unpack(ld16(ur + c), uu, T());
    unpack(ld16(g + c), gg, T());
    unpack(ld16(be + c), bb, T());
    const float sh = __shfl(dm, c / dv, kWave);  // mean_h - mean of this chunk's head
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = ((a[e] + sh) * rstd * gg[e] + bb[e]) * uu[e];
    st16(zr + c, pack(o, T()));
  }
}

// The sequence holding `row`: the largest b in [0, B) whose (clamped) start
// is <= row, found by the whole wave, 64 candidates per step.
__device__ __forceinline__ int row_sequence(const int64_t* off, int B, int64_t T, int64_t row, int lane) {
  int lo = 0, n = B;  // answer in [lo, lo + n)
  while (n > 1) {
    const int stride = (n + kWave - 1) / kWave;
    const int64_t s = lane * stride < n ? off[lo + lane * stride] : T + 1;
    const int cnt = __popcll(__ballot(min(max(s, (int64_t)0), T + 1) <= row));
    const int pick = max(cnt, 1) - 1;
    lo += pick * stride;
    n = min(stride, n - pick * stride);
  }
  return lo;
}

// Cached candidate pass: one wave per row sums the row's fp32 history-chunk
// partials of AV in chunk order (the scheduling of the attention work items
// cannot change the result), then z = (LayerNorm(AV) * g + b) * u directly
// from those fp32 values.  NC: 16-byte column groups per lane.
template <typename T, int NC>
__global__ __launch_bounds__(256) void cand_gate_kernel(const float* __restrict__ part,
                                                        const int64_t* __restrict__ off, int32_t B, int64_t Tq,
                                                        const int32_t* __restrict__ nsplit,
                                                        const T* __restrict__ u, const T* __restrict__ g,
                                                        const T* __restrict__ be, T* __restrict__ z, int K,
                                                        float eps) {
  constexpr int V = Elem<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= Tq) return;  // whole wave leaves together
  const int b = row_sequence(off, B, Tq, row, lane);
  const int ns = min(max(nsplit[b], 1), kCandMaxSplit);
  float x[NC][V];
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int e = 0; e < V; ++e) x[i][e] = 0.f;
#pragma unroll
  for (int c = 0; c < kCandMaxSplit; ++c) {
    if (c >= ns) break;
    const float* src = part + ((int64_t)c * Tq + row) * K;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int col = (lane + kWave * i) * V;
      if (col < K) {
#pragma unroll
        for (int q4 = 0; q4 < V / 4; ++q4) {
          const float4 v = *reinterpret_cast<const float4*>(src + col + 4 * q4);
          x[i][4 * q4] += v.x;
          x[i][4 * q4 + 1] += v.y;
          x[i][4 * q4 + 2] += v.z;
          x[i][4 * q4 + 3] += v.w;
        }
      }
    }
  }
  float s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if ((lane + kWave * i) * V < K)
#pragma unroll
      for (int e = 0; e < V; ++e) s1 += x[i][e];
  const float mean = wave_sum(s1) / (float)K;
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if ((lane + kWave * i) * V < K)
#pragma unroll
      for (int e = 0; e < V; ++e) s2 += (x[i][e] - mean) * (x[i][e] - mean);
  const float rstd = rsqrtf(wave_sum(s2) / (float)K + eps);
  const T* ur = u + row * K;
  T* zr = z + row * K;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int col = (lane + kWave * i) * V;
    if (col >= K) continue;
    float uu[V], gg[V], bb[V], o[V];
    unpack(ld16(ur + col), uu, T());
    unpack(ld16(g + col), gg, T());
    unpack(ld16(be + col), bb, T());
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = ((x[i][e] - mean) * rstd * gg[e] + bb[e]) * uu[e];
    st16(zr + col, pack(o, T()));
  }
}

template <typename T>
static hipError_t launch_cand_gate_t(const hstu_desc& d, const int64_t* qoff, int32_t B, int64_t Tq,
                                     const int32_t* nsplit, const float* part, const hstu_weights& w,
                                     const void* u, void* z, hipStream_t s) {
  const int K = d.num_heads * d.dv;
  const int groups = (K / Elem<T>::kVec + kWave - 1) / kWave;
  const dim3 grid((unsigned)((Tq + 3) / 4)), block(256);
#define HSTU_CG(NC_)                                                                                   \
  if (groups <= NC_) {                                                                                 \
    hipLaunchKernelGGL((cand_gate_kernel<T, NC_>), grid, block, 0, s, part, qoff, B, Tq, nsplit,        \
                       (const T*)u, (const T*)w.ln_av_g, (const T*)w.ln_av_b, (T*)z, K, d.ln_eps);    \
    return hipGetLastError();                                                                          \
  }
  HSTU_CG(1)
  HSTU_CG(2)
  HSTU_CG(4)
  HSTU_CG(8)
  HSTU_CG(16)
#undef HSTU_CG
  return hipErrorInvalidValue;
}

hipError_t launch_cand_gate(const hstu_desc& d, const int64_t* qoff, int32_t B, int64_t Tq,
                            const int32_t* nsplit, const float* part, const hstu_weights& w, const void* u,
                            void* z, hipStream_t s) {
  if (Tq == 0) return hipSuccess;
  if (d.dtype == HSTU_BF16) return launch_cand_gate_t<bf16>(d, qoff, B, Tq, nsplit, part, w, u, z, s);
  return launch_cand_gate_t<float>(d, qoff, B, Tq, nsplit, part, w, u, z, s);
}

// f2 for any dtype / width: 128 x 128 tiles.  `out` may alias `x`: each output
// element is read (residual) and written by the same thread, and nothing else
// in the kernel reads x.
template <typename T>
__global__ __launch_bounds__(256, 2) void f2_kernel(const T* x, const T* __restrict__ zin,
                                                    const T* __restrict__ w2, const T* __restrict__ b2,
                                                    T* out, int64_t M, int N, int K, int residual) {
  typedef GemmTile<T> G;
  __shared__ __attribute__((aligned(16))) T As[G::BM * G::LDK];
  __shared__ __attribute__((aligned(16))) T Bs[G::BN * G::LDK];
  const int nrow = (int)((M + G::BM - 1) / G::BM), ncol = (N + G::BN - 1) / G::BN;
  int tr, tc;
  map_tile(blockIdx.x, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G::BM;
  const int col0 = tc * G::BN;
  RowLoader<T> al{zin, row0, M, K};
  f32x16 acc[2][2];
  gemm_mainloop<T>(al, w2, col0, N, K, As, Bs, acc);

  const int lane = threadIdx.x & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int col = col0 + wn * 64 + nt * 32 + (lane & 31);
    if (col >= N) continue;
    const float bias = to_f32(b2[col]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + acc_row(wm, mt, lane, r);
        if (row < M) {
          float y = acc[mt][nt][r] + bias;
          if (residual) y += to_f32(x[row * N + col]);
          out[row * N + col] = from_f32<T>(y);
        }
      }
    }
  }
}

// f2 for bf16 with K a multiple of 64: 256 x 256 tiles, both operands copied
// straight into LDS.
__global__ __launch_bounds__(512, 2) void f2_big_kernel(const bf16* x, const bf16* __restrict__ zin,
                                                        const bf16* __restrict__ w2,
                                                        const bf16* __restrict__ b2, bf16* out, int64_t M,
                                                        int N, int K, int residual) {
  __shared__ __attribute__((aligned(16))) bf16 As0[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 As1[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Bs0[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Bs1[G2::STAGE];
  const int nrow = (int)((M + G2::BM - 1) / G2::BM), ncol = (N + G2::BN - 1) / G2::BN;
  int tr, tc;
  map_tile(blockIdx.x, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G2::BM;
  const int col0 = tc * G2::BN;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
  G2RowsA ap;
  ap.c.init(zin, row0, M, K, w, lane);
  ap.w = w;
  G2Copy bc;
  bc.init(w2, col0, N, K, w, lane);
  f32x16 acc[2][4];
  g2_mainloop<true>(ap, bc, K, As0, As1, Bs0, Bs1, acc);

  // Epilogue through LDS (the operand stages are free once every wave is
  // past its last MFMA read): residual tile in, + acc + b2 in place, rows out.
  // Every x element of the tile is read before any element of out is
  // written, so out may alias x.
  __syncthreads();
  const G2Quarters qs{As0, As1, Bs0, Bs1};
  if (residual) {
    g2_out_load(x, row0, M, col0, N, N, qs, tid, w);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  bf16* const yq = qs[wm];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int ct = wn * 128 + nt * 32 + (lane & 31);
    const float bias = col0 + ct < N ? (float)b2[col0 + ct] : 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        bf16* p = yq + g2_out_off(g2_out_row(mt, lane, r), ct);
        float y = acc[mt][nt][r] + bias;
        if (residual) y += (float)*p;
        *p = (bf16)y;
      }
  }
  __syncthreads();
  const int col = col0 + 8 * g2_out_chunk(tid);
  if (col < N) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = i * G2::NT + tid;
      const int64_t row = row0 + (s >> 5);
      if (row < M) st16(out + row * N + col, ld16(qs[i >> 2] + (s & (4 * G2::NT - 1)) * 8));
    }
  }
}

hipError_t launch_gate(const hstu_desc& d, int64_t T, const hstu_weights& w, const void* u,
                       const void* av, const float* stats, void* z, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL(gate_kernel<bf16>, grid, block, 0, s, (const bf16*)av, (const bf16*)u, stats,
                       (const bf16*)w.ln_av_g, (const bf16*)w.ln_av_b, (bf16*)z, T, d.num_heads, d.dv,
                       d.ln_eps);
  else
    hipLaunchKernelGGL(gate_kernel<float>, grid, block, 0, s, (const float*)av, (const float*)u, stats,
                       (const float*)w.ln_av_g, (const float*)w.ln_av_b, (float*)z, T, d.num_heads,
                       d.dv, d.ln_eps);
  return hipGetLastError();
}

hipError_t launch_f2(const hstu_desc& d, const void* x, int64_t T, const hstu_weights& w,
                     const void* z, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int N = d.d_model, K = d.num_heads * d.dv;
  const int res = (d.flags & HSTU_RESIDUAL) ? 1 : 0;
  if (d.dtype == HSTU_BF16 && K % G2::BK == 0) {
    const int64_t nr = (T + G2::BM - 1) / G2::BM, nc = (N + G2::BN - 1) / G2::BN;
    hipLaunchKernelGGL(f2_big_kernel, dim3((unsigned)(nr * nc)), dim3(G2::NT), 0, s, (const bf16*)x,
                       (const bf16*)z, (const bf16*)w.w2, (const bf16*)w.b2, (bf16*)out, T, N, K, res);
    return hipGetLastError();
  }
  const int64_t nrow = (T + 127) / 128, ncol = (N + 127) / 128;
  dim3 grid((unsigned)(nrow * ncol)), block(256);
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL(f2_kernel<bf16>, grid, block, 0, s, (const bf16*)x, (const bf16*)z,
                       (const bf16*)w.w2, (const bf16*)w.b2, (bf16*)out, T, N, K, res);
  else
    hipLaunchKernelGGL(f2_kernel<float>, grid, block, 0, s, (const float*)x, (const float*)z,
                       (const float*)w.w2, (const float*)w.b2, (float*)out, T, N, K, res);
  return hipGetLastError();
}

}  // namespace hstu
