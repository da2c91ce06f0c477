// Stage 3: Y = f2(LayerNorm(AV) * U) + b2 (+ x) — page "4.4 Scaling
// Recommendation Models", section "Generative Recommenders and HSTU" (third
// layer equation; gating in place of an FFN) and section "Code" (LayerNorm over
// the merged heads, multiply by u, f2, residual add); page "HSTU: The First
// Exploration of the Scaling Law", 7.1.4 Innovation 1 (LayerNorm(AV) * U).
//
// One fused kernel: the A operand of the f2 GEMM is produced on the fly from
// the per-head-centred AV, the fp32 per-(row, head) statistics written by the
// attention kernel, the LayerNorm affine and U; bias and residual are added in
// the epilogue.  Row statistics are merged from the H head partials with the
// parallel-variance formula: mean = avg_h mean_h,
// M2 = sum_h M2_h + dv * sum_h (mean_h - mean)^2, so no bf16-rounded value ever
// enters a variance.
#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace hstu {

template <typename T>
struct GateLoader {
  const T* __restrict__ av;
  const T* __restrict__ u;
  const T* __restrict__ g;
  const T* __restrict__ be;
  T* __restrict__ z_out;  // optional copy of the produced operand
  const float* __restrict__ stats;  // [M, H, 2] per-head mean, M2
  const float* s_mean;    // [BM] LDS: mean of the merged row
  const float* s_rstd;    // [BM] LDS: 1 / sqrt(var + eps)
  int64_t row0, M;
  int K, H, dv;
  __device__ __forceinline__ uint4 operator()(int k0, int r, int kc) const {
    constexpr int V = Elem<T>::kVec;
    const int64_t row = row0 + r;
    const int k = k0 + kc;
    if (row >= M || k >= K) return make_uint4(0, 0, 0, 0);
    float a[V], uu[V], gg[V], bb[V], z[V];
    unpack(ld16(av + row * K + k), a, T());
    unpack(ld16(u + row * K + k), uu, T());
    unpack(ld16(g + k), gg, T());
    unpack(ld16(be + k), bb, T());
    const float rs = s_rstd[r], sh = stats[(row * H + k / dv) * 2] - s_mean[r];
#pragma unroll
    for (int e = 0; e < V; ++e) z[e] = ((a[e] + sh) * rs * gg[e] + bb[e]) * uu[e];
    uint4 out = pack(z, T());
    if (z_out) st16(z_out + row * K + k, out);
    return out;
  }
};

// `out` may alias `x`: each output element is read (residual) and written by
// the same thread, and nothing else in the kernel reads x.
template <typename T>
__global__ __launch_bounds__(256, 2) void out_kernel(const T* x, const T* __restrict__ w2,
                                                     const T* __restrict__ b2, const T* __restrict__ g,
                                                     const T* __restrict__ be, const T* __restrict__ u,
                                                     const T* __restrict__ av,
                                                     const float* __restrict__ stats,
                                                     T* out, T* __restrict__ z_out,
                                                     int64_t M, int N, int H, int dv, float eps,
                                                     int residual) {
  typedef GemmTile<T> G;
  __shared__ __attribute__((aligned(16))) T As[G::BM * G::LDK];
  __shared__ __attribute__((aligned(16))) T Bs[G::BN * G::LDK];
  __shared__ float s_mean[G::BM], s_rstd[G::BM];
  const int K = H * dv;
  const int nrow = (int)((M + G::BM - 1) / G::BM), ncol = (N + G::BN - 1) / G::BN;
  int tr, tc;
  map_tile(blockIdx.x, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G::BM;
  const int col0 = tc * G::BN;

  // Row statistics of the merged heads.
  for (int r = threadIdx.x; r < G::BM; r += 256) {
    const int64_t row = row0 + r;
    float mean = 0.f, rstd = 0.f;
    if (row < M) {
      const float* st = stats + row * H * 2;
      for (int h = 0; h < H; ++h) mean += st[2 * h];
      mean /= (float)H;
      float m2 = 0.f;
      for (int h = 0; h < H; ++h) {
        const float dm = st[2 * h] - mean;
        m2 += st[2 * h + 1] + (float)dv * dm * dm;
      }
      rstd = rsqrtf(m2 / (float)K + eps);
    }
    s_mean[r] = mean;
    s_rstd[r] = rstd;
  }
  __syncthreads();

  GateLoader<T> al{av, u, g, be, tc == 0 ? z_out : nullptr, stats, s_mean, s_rstd, row0, M, K, H, dv};
  f32x16 acc[2][2];
  gemm_mainloop<T>(al, w2, col0, N, K, As, Bs, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
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

hipError_t launch_out(const hstu_desc& d, const void* x, int64_t T, const hstu_weights& w,
                      const void* u, const void* av, const float* stats, void* out, void* z_out,
                      hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int N = d.d_model;
  const int64_t nrow = (T + 127) / 128, ncol = (N + 127) / 128;
  dim3 grid((unsigned)(nrow * ncol)), block(256);
  const int res = (d.flags & HSTU_RESIDUAL) ? 1 : 0;
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL(out_kernel<bf16>, grid, block, 0, s, (const bf16*)x, (const bf16*)w.w2,
                       (const bf16*)w.b2, (const bf16*)w.ln_av_g, (const bf16*)w.ln_av_b,
                       (const bf16*)u, (const bf16*)av, stats, (bf16*)out, (bf16*)z_out, T, N,
                       d.num_heads, d.dv, d.ln_eps, res);
  else
    hipLaunchKernelGGL(out_kernel<float>, grid, block, 0, s, (const float*)x, (const float*)w.w2,
                       (const float*)w.b2, (const float*)w.ln_av_g, (const float*)w.ln_av_b,
                       (const float*)u, (const float*)av, stats, (float*)out, (float*)z_out, T, N,
                       d.num_heads, d.dv, d.ln_eps, res);
  return hipGetLastError();
}

}  // namespace hstu
