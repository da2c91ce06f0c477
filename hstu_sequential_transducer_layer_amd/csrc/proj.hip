// Stage 1: U, V, Q, K = Split(SiLU(f1(x~))) — page "4.4 Scaling
// Recommendation Models", section "Generative Recommenders and HSTU" (first
// layer equation) and section "Code" (f1 then SiLU, chunked u | v | q | k,
// head h owning contiguous columns of each chunk).
//
// One MFMA GEMM over all packed rows of the jagged batch (the rows of a jagged
// batch are just tokens here), with +b1 and SiLU in the epilogue, and the
// result scattered straight into the layouts the attention kernel streams:
//   U [T, H*dv] row-major, V [H, T, dv], Q [H, T, dqk], K [H, T, dqk];
// for training also the pre-activation x~ W1^T + b1 [T, N1] row-major, which
// the backward needs for the SiLU derivative.
#include "common.h"
#include "gemm.h"
#include "gemm2.h"
#include "kernels.h"

namespace hstu {

template <typename T>
__global__ __launch_bounds__(256, 2) void proj_kernel(const T* __restrict__ xn, const T* __restrict__ w1,
                                                      const T* __restrict__ b1, T* __restrict__ u,
                                                      T* __restrict__ v, T* __restrict__ q,
                                                      T* __restrict__ k, T* __restrict__ pre, int64_t M,
                                                      int N, int K, int H, int dqk, int dv) {
  typedef GemmTile<T> G;
  __shared__ __attribute__((aligned(16))) T As[G::BM * G::LDK];
  __shared__ __attribute__((aligned(16))) T Bs[G::BN * G::LDK];
  const int nrow = (int)((M + G::BM - 1) / G::BM), ncol = (N + G::BN - 1) / G::BN;
  int tr, tc;
  map_tile(blockIdx.x, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G::BM;
  const int col0 = tc * G::BN;
  RowLoader<T> al{xn, row0, M, K};
  f32x16 acc[2][2];
  gemm_mainloop<T>(al, w1, col0, N, K, As, Bs, acc);

  const int lane = threadIdx.x & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
  const int HDV = H * dv, HDQ = H * dqk;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int cb = col0 + wn * 64 + nt * 32;  // first column of this 32-wide tile
    if (cb >= N) continue;
    const int col = cb + (lane & 31);
    const float bias = to_f32(b1[col]);
    // Destination of this tile's columns: all 32 lie in one chunk and one head.
    T* base;
    int64_t rstride;
    if (cb < HDV) {
      base = u + col;
      rstride = HDV;
    } else if (cb < 2 * HDV) {
      const int c = cb - HDV, h = c / dv;
      base = v + (int64_t)h * M * dv + (c % dv) + (lane & 31);
      rstride = dv;
    } else if (cb < 2 * HDV + HDQ) {
      const int c = cb - 2 * HDV, h = c / dqk;
      base = q + (int64_t)h * M * dqk + (c % dqk) + (lane & 31);
      rstride = dqk;
    } else {
      const int c = cb - 2 * HDV - HDQ, h = c / dqk;
      base = k + (int64_t)h * M * dqk + (c % dqk) + (lane & 31);
      rstride = dqk;
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + acc_row(wm, mt, lane, r);
        if (row < M) {
          base[row * rstride] = from_f32<T>(silu(acc[mt][nt][r] + bias));
          if (pre) pre[row * N + col] = from_f32<T>(acc[mt][nt][r] + bias);
        }
      }
    }
  }
}

// Destination of output columns [cb, cb + 32): base pointer (already offset by
// the lane's column) and row stride.  All 32 columns lie in one chunk of
// U | V | Q | K and in one head, since every block and head width is a
// multiple of 32.
template <typename T>
__device__ __forceinline__ T* proj_dst(int cb, int lane, T* u, T* v, T* q, T* k, int64_t M, int H,
                                       int dqk, int dv, int64_t& rstride) {
  const int HDV = H * dv, HDQ = H * dqk;
  if (cb < HDV) {
    rstride = HDV;
    return u + cb + (lane & 31);
  }
  if (cb < 2 * HDV) {
    const int c = cb - HDV, h = c / dv;
    rstride = dv;
    return v + (int64_t)h * M * dv + (c % dv) + (lane & 31);
  }
  if (cb < 2 * HDV + HDQ) {
    const int c = cb - 2 * HDV, h = c / dqk;
    rstride = dqk;
    return q + (int64_t)h * M * dqk + (c % dqk) + (lane & 31);
  }
  const int c = cb - 2 * HDV - HDQ, h = c / dqk;
  rstride = dqk;
  return k + (int64_t)h * M * dqk + (c % dqk) + (lane & 31);
}

// Large-tile bf16 version (K a multiple of 64): 256 x 256 tiles, operands
// copied straight into LDS.  PRE: also the pre-activation (a compile-time
// choice: as a run-time branch it costs the epilogue ~190 spilled registers).
template <bool PRE>
__global__ __launch_bounds__(512, 2) void proj2_kernel(const bf16* __restrict__ xn, const bf16* __restrict__ w1,
                                                       const bf16* __restrict__ b1, bf16* __restrict__ u,
                                                       bf16* __restrict__ v, bf16* __restrict__ q,
                                                       bf16* __restrict__ k, bf16* __restrict__ pre, int64_t M,
                                                       int N, int K, int H, int dqk, int dv) {
  __shared__ __attribute__((aligned(16))) bf16 As0[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 As1[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Bs0[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Bs1[G2::STAGE];
  const int nrow = (int)((M + G2::BM - 1) / G2::BM), ncol = (N + G2::BN - 1) / G2::BN;
  int tr, tc;
  map_tile(blockIdx.x, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G2::BM;
  const int col0 = tc * G2::BN;
  const int lane = threadIdx.x & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
  G2RowsA ap;
  ap.c.init(xn, row0, M, K, w, lane);
  ap.w = w;
  G2Copy bc;
  bc.init(w1, col0, N, K, w, lane);
  f32x16 acc[2][4];
  g2_mainloop<true>(ap, bc, K, As0, As1, Bs0, Bs1, acc);

  // Epilogue through LDS: SiLU(acc + b1) into the staged tile, then rows out
  // with 16-byte stores (a 16-byte chunk never straddles a head or a chunk of
  // U | V | Q | K).  With pre, acc + b1 goes the same way first, into the
  // row-major [M, N] pre-activation.
  __syncthreads();
  const G2Quarters qs{As0, As1, Bs0, Bs1};
  bf16* const yq = qs[wm];
  float bias[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int ct = wn * 128 + nt * 32 + (lane & 31);
    bias[nt] = col0 + ct < N ? (float)b1[col0 + ct] : 0.f;
  }
  const int col = col0 + 8 * g2_out_chunk(threadIdx.x);
  if constexpr (PRE) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int ct = wn * 128 + nt * 32 + (lane & 31);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) yq[g2_out_off(g2_out_row(mt, lane, r), ct)] = (bf16)(acc[mt][nt][r] + bias[nt]);
    }
    __syncthreads();
    if (col < N) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int s = i * G2::NT + threadIdx.x;
        const int64_t row = row0 + (s >> 5);
        if (row < M) st16(pre + row * N + col, ld16(qs[i >> 2] + (s & (4 * G2::NT - 1)) * 8));
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int ct = wn * 128 + nt * 32 + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        yq[g2_out_off(g2_out_row(mt, lane, r), ct)] = (bf16)silu(acc[mt][nt][r] + bias[nt]);
  }
  __syncthreads();
  if (col < N) {
    int64_t rstride;
    bf16* base = proj_dst(col & ~31, 0, u, v, q, k, M, H, dqk, dv, rstride) + (col & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = i * G2::NT + threadIdx.x;
      const int64_t row = row0 + (s >> 5);
      if (row < M) st16(base + row * rstride, ld16(qs[i >> 2] + (s & (4 * G2::NT - 1)) * 8));
    }
  }
}

hipError_t launch_proj(const hstu_desc& d, const void* xn, int64_t T, const void* w1,
                       const void* b1, void* u, void* v, void* q, void* k, void* pre, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int N = 2 * d.num_heads * (d.dqk + d.dv), K = d.d_model;
  const int64_t nr = (T + G2::BM - 1) / G2::BM, nc = (N + G2::BN - 1) / G2::BN;
  // 256 x 256 tiles unless they would leave most compute units idle; a small
  // problem (a candidate micro-batch) runs 4x as many 128 x 128 tiles instead
  if (d.dtype == HSTU_BF16 && K % G2::BK == 0 && nr * nc >= kG2MinTiles) {
    if (pre)
      hipLaunchKernelGGL(proj2_kernel<true>, dim3((unsigned)(nr * nc)), dim3(G2::NT), 0, s, (const bf16*)xn,
                         (const bf16*)w1, (const bf16*)b1, (bf16*)u, (bf16*)v, (bf16*)q, (bf16*)k, (bf16*)pre,
                         T, N, K, d.num_heads, d.dqk, d.dv);
    else
      hipLaunchKernelGGL(proj2_kernel<false>, dim3((unsigned)(nr * nc)), dim3(G2::NT), 0, s, (const bf16*)xn,
                         (const bf16*)w1, (const bf16*)b1, (bf16*)u, (bf16*)v, (bf16*)q, (bf16*)k, nullptr,
                         T, N, K, d.num_heads, d.dqk, d.dv);
    return hipGetLastError();
  }
  const int64_t nrow = (T + 127) / 128, ncol = (N + 127) / 128;
  dim3 grid((unsigned)(nrow * ncol)), block(256);
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL(proj_kernel<bf16>, grid, block, 0, s, (const bf16*)xn, (const bf16*)w1,
                       (const bf16*)b1, (bf16*)u, (bf16*)v, (bf16*)q, (bf16*)k, (bf16*)pre, T, N, K,
                       d.num_heads, d.dqk, d.dv);
  else
    hipLaunchKernelGGL(proj_kernel<float>, grid, block, 0, s, (const float*)xn, (const float*)w1,
                       (const float*)b1, (float*)u, (float*)v, (float*)q, (float*)k, (float*)pre, T, N, K,
                       d.num_heads, d.dqk, d.dv);
  return hipGetLastError();
}

}  // namespace hstu
