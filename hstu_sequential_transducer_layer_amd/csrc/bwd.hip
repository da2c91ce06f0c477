// The layer backward around the attention (row f2): the gradients of
//   x~ = LayerNorm_in(x);  u|v|q|k = SiLU(x~ W1^T + b1);
//   Z = (LayerNorm_av(AV) * g + b) * U;  Y = Z W2^T + b2 (+ x)
// (page "4.4 Scaling Recommendation Models", "Generative Recommenders and
// HSTU" first and third layer equations and the "Code" sketch; page "HSTU:
// The First Exploration of the Scaling Law", 7.1.4 Innovation 1).
// Kernels:
//   transpose_kernel      [R, C] -> [C, Rp] in the layer dtype, columns past R zero
//   gemm_nt_f32_kernel    C = A B^T with fp32 output (128 x 128 tiles, MFMA)
//   colsum_rows_kernel, colsum_chunks_kernel: column sums, in two
//                         deterministic stages
//   gate_bwd_kernel       one wave per row: dU, dL/dAV, and the per-row terms
//                         of the LayerNorm_av parameter gradients
//   gemm_silu_bwd_kernel  pre = x~ W1^T on MFMA, kept on chip (LDS); dpre =
//                         d(u|v|q|k) * SiLU'(pre + b1) and db1's row-chunk sums
//   ln_bwd_kernel         one wave per row: dx through LayerNorm_in (+ dY)
#include <type_traits>

#include "common.h"
#include "gemm.h"
#include "gemm2.h"
#include "kernels.h"

namespace hstu {

// Eight consecutive elements (16-byte aligned) to and from fp32 registers:
// one 16-byte access for bf16, two for fp32.
__device__ __forceinline__ void load8(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16* p, float (&f)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const bf16* e = reinterpret_cast<const bf16*>(&raw);
#pragma unroll
  for (int q = 0; q < 8; ++q) f[q] = to_f32(e[q]);
}
__device__ __forceinline__ void store8(float* p, const float (&f)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float (&f)[8]) {
  bf16 e[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) e[q] = from_f32<bf16>(f[q]);
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(e);
}

// dst[c][r] = src[r][c] (zero for r >= R) for r < Rp, c < C, through a 64 x 64
// LDS tile; 16-byte loads along the source rows and 16-byte stores along the
// destination rows.  C, Rp multiples of 16 / sizeof(T).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int64_t R, int64_t C, int64_t Rp,
                                                        T* __restrict__ dst) {
  constexpr int V = 16 / (int)sizeof(T), VPR = 64 / V, PAD = 4 / (int)sizeof(T);
  __shared__ T tile[64][64 + PAD];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 64 * VPR / 256; ++k) {
    const int idx = t + 256 * k, i = idx / VPR, j = idx % VPR;
    const int64_t r = r0 + i, c = c0 + (int64_t)j * V;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R && c < C) v = *reinterpret_cast<const uint4*>(src + r * C + c);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int q = 0; q < V; ++q) tile[i][j * V + q] = e[q];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 64 * VPR / 256; ++k) {
    const int idx = t + 256 * k, cc = idx / VPR, m = idx % VPR;
    const int64_t c = c0 + cc, r = r0 + (int64_t)m * V;
    uint4 v;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int q = 0; q < V; ++q) e[q] = tile[m * V + q][cc];
    if (c < C && r < Rp) *reinterpret_cast<uint4*>(dst + c * Rp + r) = v;
  }
}

// Split over K: workgroup (tile, s) multiplies columns [s kc, (s + 1) kc) and
// writes its partial product to C + s M N (summed afterwards in s order).
template <typename T>
__global__ __launch_bounds__(256, 2) void gemm_nt_f32_kernel(const T* __restrict__ A, const T* __restrict__ Bm,
                                                             float* __restrict__ C, int64_t M, int N, int K,
                                                             int kc) {
  typedef GemmTile<T> G;
  __shared__ __attribute__((aligned(16))) T As[G::BM * G::LDK];
  __shared__ __attribute__((aligned(16))) T Bs[G::BN * G::LDK];
  const int nrow = (int)((M + G::BM - 1) / G::BM), ncol = (N + G::BN - 1) / G::BN;
  const int tiles = nrow * ncol, split = blockIdx.x / tiles;
  int tr, tc;
  map_tile(blockIdx.x - split * tiles, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G::BM;
  const int col0 = tc * G::BN;
  const int k0 = split * kc, kn = min(kc, K - k0);
  C += (int64_t)split * M * N;
  RowLoader<T> al{A + k0, row0, M, kn, K};
  f32x16 acc[2][2];
  gemm_mainloop<T>(al, Bm + k0, col0, N, kn, As, Bs, acc, K);
  const int lane = threadIdx.x & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int col = col0 + wn * 64 + nt * 32 + (lane & 31);
    if (col >= N) continue;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + acc_row(wm, mt, lane, r);
        if (row < M) C[row * N + col] = acc[mt][nt][r];
      }
  }
}

// Column sums in two deterministic stages.
// Stage 1: dst[chunk][c] = sum of src rows [chunk * kColRows, ...) for column
// c; each lane owns four adjacent columns (one vector load per row) and keeps
// four rows' loads in flight.  C is a multiple of 4.
constexpr int kColRows = 128;
template <typename TIn>
__global__ __launch_bounds__(256) void colsum_rows_kernel(const TIn* __restrict__ src, int64_t R, int64_t C,
                                                          float* __restrict__ dst) {
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= C) return;
  const int64_t r0 = (int64_t)blockIdx.y * kColRows, r1 = min(r0 + kColRows, R);
  float4 acc[4] = {};
  auto load4 = [&](int64_t r) __attribute__((always_inline)) {
    const TIn* p = src + r * C + c;
    if constexpr (sizeof(TIn) == 4) {
      return *reinterpret_cast<const float4*>(p);
    } else {
      const uint2 raw = *reinterpret_cast<const uint2*>(p);
      const TIn* e = reinterpret_cast<const TIn*>(&raw);
      return make_float4(to_f32(e[0]), to_f32(e[1]), to_f32(e[2]), to_f32(e[3]));
    }
  };
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 v = load4(r + u);
      acc[u].x += v.x;
      acc[u].y += v.y;
      acc[u].z += v.z;
      acc[u].w += v.w;
    }
  }
  for (; r < r1; ++r) {  // at most three rows left
    const float4 v = load4(r);
    acc[0].x += v.x;
    acc[0].y += v.y;
    acc[0].z += v.z;
    acc[0].w += v.w;
  }
  float4 t;
  t.x = (acc[0].x + acc[1].x) + (acc[2].x + acc[3].x);
  t.y = (acc[0].y + acc[1].y) + (acc[2].y + acc[3].y);
  t.z = (acc[0].z + acc[1].z) + (acc[2].z + acc[3].z);
  t.w = (acc[0].w + acc[1].w) + (acc[2].w + acc[3].w);
  *reinterpret_cast<float4*>(dst + blockIdx.y * C + c) = t;
}

// Stage 2: dst[c] = sum over chunk < nchunks of part[chunk][c].  One
// workgroup per 64 columns; its 16 waves take every 16th chunk, then the 16
// partial sums are added in wave order.
constexpr int kColGroups = 16;
__global__ __launch_bounds__(64 * kColGroups) void colsum_chunks_kernel(const float* __restrict__ part,
                                                                        int64_t nchunks, int64_t C,
                                                                        float* __restrict__ dst) {
  __shared__ float red[kColGroups][64];
  const int t = threadIdx.x, col = t & 63, g = t >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + col;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (c < C) {
    int64_t k = g;
    for (; k + 3 * kColGroups < nchunks; k += 4 * kColGroups) {
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += part[(k + u * kColGroups) * C + c];
    }
#pragma unroll
    for (int u = 0; u < 3; ++u)
      if (k + u * kColGroups < nchunks) acc[u] += part[(k + u * kColGroups) * C + c];
  }
  red[g][col] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (g != 0 || c >= C) return;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kColGroups; ++i) sum += red[i][col];
  dst[c] = sum;
}

// Rows of the LayerNorm backward kernels: eight consecutive rows per wave, 32
// per workgroup.  The per-row terms of the LayerNorm parameters' gradients
// are summed over a workgroup's rows in a fixed order (each wave over its
// rows in order, then the four waves in order) into one partial row per
// workgroup, which colsum_chunks_kernel then sums over the workgroups; so
// the [T, columns] term arrays are never written.  Columns (H * dv, d_model):
// a multiple of 8, at most kBwdRowCols.
// NC = ceil(columns / 512) chunks of 8 columns per lane: the per-lane
// accumulators of the parameters' gradients are sized for the layer's width.
constexpr int kRowsPerWave = 8, kChunkRows = 4 * kRowsPerWave, kBwdRowCols = 2048;

// Runs f(std::integral_constant<int, NC>) for the chunk count of K columns.
template <typename F>
static void with_chunks(int K, F f) {
  if (K <= 512)
    f(std::integral_constant<int, 1>{});
  else if (K <= 1024)
    f(std::integral_constant<int, 2>{});
  else
    f(std::integral_constant<int, 4>{});
}

// The partial rows of the two terms accumulated by each wave (lane: columns
// lane * 8 + 512 j .. + 7): written to LDS, then added in wave order.
template <int NC>
__device__ __forceinline__ void chunk_partials(const float (&ga)[NC][8], const float (&ba)[NC][8], int K, float* red,
                                               float* __restrict__ gpart, float* __restrict__ bpart) {
  const int lane = threadIdx.x & 63, w = wave_id();
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = lane * 8 + 512 * j;
    if (c < K) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        red[w * K + c + e] = ga[j][e];
        red[(4 + w) * K + c + e] = ba[j][e];
      }
    }
  }
  __syncthreads();
  const int64_t o = (int64_t)blockIdx.x * K;
  for (int c = threadIdx.x; c < K; c += 256) {
    gpart[o + c] = ((red[c] + red[K + c]) + red[2 * K + c]) + red[3 * K + c];
    bpart[o + c] = ((red[4 * K + c] + red[5 * K + c]) + red[6 * K + c]) + red[7 * K + c];
  }
}

// One wave per row.  Recomputes the LayerNorm of AV from the attention's
// per-head statistics (the forward gate's merge), then
//   n^ = (AV - mean) * rstd,  dn = dZ * U,  dn^ = dn * g
//   dU = dZ * (n^ g + b),  dAV = rstd (dn^ - mean(dn^) - n^ mean(dn^ n^))
// and the workgroup's partial sums of dn * n^ and dn (the terms of dg and db).
template <typename T, int NC>
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ dz, const T* __restrict__ u,
                                                       const T* __restrict__ av, const float* __restrict__ stats,
                                                       const T* __restrict__ g, const T* __restrict__ be,
                                                       int64_t M, int H, int dv, float eps, int64_t n1,
                                                       const T* __restrict__ pre, T* __restrict__ dpre,
                                                       T* __restrict__ dav, float* __restrict__ gpart,
                                                       float* __restrict__ bpart) {
  // a lane takes 8 consecutive columns of one head per step (dv a multiple of 8)
  extern __shared__ float red[];  // [2][4 waves][K]
  const int lane = threadIdx.x & 63, w = wave_id();
  const int K = H * dv;
  float ga[NC][8], ba[NC][8];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ga[j][e] = ba[j][e] = 0.f;
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t row = (int64_t)blockIdx.x * kChunkRows + w * kRowsPerWave + i;
    if (row >= M) break;  // wave-uniform
    const float2 st = lane < H ? reinterpret_cast<const float2*>(stats)[row * H + lane] : make_float2(0.f, 0.f);
    const float mean = wave_sum(st.x) / (float)H;
    const float dm = st.x - mean;
    const float m2 = wave_sum(lane < H ? st.y + (float)dv * dm * dm : 0.f);
    const float rstd = rsqrtf(m2 / (float)K + eps);
    const int64_t o = row * K;
    float s1 = 0.f, s2 = 0.f;
    float a8[8], z8[8], u8[8], g8[8];
    for (int c = lane * 8; c < K; c += 8 * kWave) {
      const float off = __shfl(dm, c / dv, kWave);
      load8(av + o + c, a8);
      load8(dz + o + c, z8);
      load8(u + o + c, u8);
      load8(g + c, g8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float nh = (a8[e] + off) * rstd;
        const float dnh = z8[e] * u8[e] * g8[e];
        s1 += dnh;
        s2 += dnh * nh;
      }
    }
    const float m1 = wave_sum(s1) / (float)K, mm = wave_sum(s2) / (float)K;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = lane * 8 + 512 * j;
      if (c >= K) break;
      const float off = __shfl(dm, c / dv, kWave);
      float b8[8], p8[8], o_du[8], o_dav[8];
      load8(av + o + c, a8);
      load8(dz + o + c, z8);
      load8(u + o + c, u8);
      load8(g + c, g8);
      load8(be + c, b8);
      load8(pre + row * n1 + c, p8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float nh = (a8[e] + off) * rstd;
        const float dn = z8[e] * u8[e];
        o_du[e] = z8[e] * (nh * g8[e] + b8[e]) * silu_grad(p8[e]);
        o_dav[e] = rstd * (dn * g8[e] - m1 - nh * mm);
        ga[j][e] += dn * nh;
        ba[j][e] += dn;
      }
      store8(dpre + row * n1 + c, o_du);
      store8(dav + o + c, o_dav);
    }
  }
  chunk_partials(ga, ba, K, red, gpart, bpart);
}


// One wave per row (eight consecutive rows per wave, as above).  With the
// input LayerNorm: x^ = (x - mean) rstd,
// dx = rstd (dxn g - mean(dxn g) - x^ mean(dxn g x^)); else dx = dxn.  Plus dY
// for the residual.  With the LayerNorm, the workgroup's partial sums of
// dxn * x^ and dxn (the terms of its gain's and offset's gradients).
template <typename T, int NC>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const T* __restrict__ x, const float* __restrict__ dxn,
                                                     const T* __restrict__ g, const T* __restrict__ dy, int64_t M,
                                                     int d, float eps, int norm, int residual, T* __restrict__ dx,
                                                     float* __restrict__ gpart, float* __restrict__ bpart) {
  // a lane takes 8 consecutive columns per step (16-byte accesses for bf16),
  // d a multiple of 8
  extern __shared__ float red[];  // [2][4 waves][d]
  const int lane = threadIdx.x & 63, w = wave_id();
  float ga[NC][8], ba[NC][8];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ga[j][e] = ba[j][e] = 0.f;
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t row = (int64_t)blockIdx.x * kChunkRows + w * kRowsPerWave + i;
    if (row >= M) break;  // wave-uniform
    const int64_t o = row * d;
    float mean = 0.f, rstd = 1.f, m1 = 0.f, mm = 0.f;
    float xv[8], gv[8], dv8[8];
    if (norm) {
      float sx = 0.f;
      for (int c = lane * 8; c < d; c += 8 * kWave) {
        load8(x + o + c, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) sx += xv[e];
      }
      mean = wave_sum(sx) / (float)d;
      float v = 0.f;
      for (int c = lane * 8; c < d; c += 8 * kWave) {
        load8(x + o + c, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = xv[e] - mean;
          v += t * t;
        }
      }
      rstd = rsqrtf(wave_sum(v) / (float)d + eps);
      float s1 = 0.f, s2 = 0.f;
      for (int c = lane * 8; c < d; c += 8 * kWave) {
        load8(x + o + c, xv);
        load8(g + c, gv);
        load8(dxn + o + c, dv8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[e] - mean) * rstd;
          const float t = dv8[e] * gv[e];
          s1 += t;
          s2 += t * xh;
        }
      }
      m1 = wave_sum(s1) / (float)d;
      mm = wave_sum(s2) / (float)d;
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = lane * 8 + 512 * j;
      if (c >= d) break;
      float r[8], yv[8];
      load8(dxn + o + c, dv8);
      if (norm) {
        load8(x + o + c, xv);
        load8(g + c, gv);
      }
      if (residual) load8(dy + o + c, yv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (norm) {
          const float xh = (xv[e] - mean) * rstd;
          r[e] = rstd * (dv8[e] * gv[e] - m1 - xh * mm);
          ga[j][e] += dv8[e] * xh;
          ba[j][e] += dv8[e];
        } else {
          r[e] = dv8[e];
        }
        if (residual) r[e] += yv[e];
      }
      store8(dx + o + c, r);
    }
  }
  chunk_partials(ga, ba, d, red, gpart, bpart);
}

template <typename T>
static hipError_t colsum_t(const T* src, int64_t R, int64_t C, float* tmp, float* dst, hipStream_t s) {
  if (C % 4 != 0) return hipErrorInvalidValue;
  const int64_t chunks = (R + kColRows - 1) / kColRows;
  if (chunks > 0)
    hipLaunchKernelGGL(colsum_rows_kernel<T>, dim3((unsigned)((C / 4 + 255) / 256), (unsigned)chunks), dim3(256), 0, s,
                       src, R, C, tmp);
  hipLaunchKernelGGL(colsum_chunks_kernel, dim3((unsigned)((C + 63) / 64)), dim3(64 * kColGroups), 0, s,
                     (const float*)tmp, chunks, C, dst);
  return hipGetLastError();
}

size_t colsum_tmp_bytes(int64_t R, int64_t C) {
  return (size_t)((R + kColRows - 1) / kColRows + 1) * (size_t)C * sizeof(float);
}

hipError_t launch_colsum(hstu_dtype dt_in, bool in_f32, const void* src, int64_t R, int64_t C, float* tmp, float* dst,
                         hipStream_t s) {
  if (in_f32) return colsum_t<float>((const float*)src, R, C, tmp, dst, s);
  if (dt_in == HSTU_BF16) return colsum_t<bf16>((const bf16*)src, R, C, tmp, dst, s);
  return colsum_t<float>((const float*)src, R, C, tmp, dst, s);
}

hipError_t launch_transpose(hstu_dtype dt, const void* src, int64_t R, int64_t C, int64_t Rp, void* dst,
                            hipStream_t s) {
  if (R == 0 && Rp == 0) return hipSuccess;
  const int64_t vec = dt == HSTU_BF16 ? 8 : 4;
  if (C % vec != 0 || Rp % vec != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((Rp + 63) / 64), (unsigned)((C + 63) / 64)), block(256);
  if (dt == HSTU_BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, block, 0, s, (const bf16*)src, R, C, Rp, (bf16*)dst);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, (const float*)src, R, C, Rp, (float*)dst);
  return hipGetLastError();
}

// dst[i] = sum over s < S of part[s * n + i], in s order.
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int64_t n, int S,
                                                        float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * n + i];
  dst[i] = v;
}

// The same product on the forward's 256 x 256 core (bf16, every K chunk a
// multiple of 64): operands copied straight into LDS, fp32 results stored from
// the accumulators (32 consecutive columns per row and store instruction).
// Split s covers k in [s * kc, min((s + 1) * kc, K)) and writes C + s * M * N;
// within a split the k16 steps run in ascending order, as in
// gemm_nt_f32_kernel.
__global__ __launch_bounds__(512, 2) void gemm_nt_f32_big_kernel(const bf16* __restrict__ A,
                                                                 const bf16* __restrict__ Bm, float* __restrict__ C,
                                                                 int64_t M, int N, int K, int kc) {
  __shared__ __attribute__((aligned(16))) bf16 As0[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 As1[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Bs0[G2::STAGE];
  __shared__ __attribute__((aligned(16))) bf16 Bs1[G2::STAGE];
  const int nrow = (int)((M + G2::BM - 1) / G2::BM), ncol = (N + G2::BN - 1) / G2::BN;
  const int tiles = nrow * ncol, split = blockIdx.x / tiles;
  int tr, tc;
  map_tile(blockIdx.x - split * tiles, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G2::BM;
  const int col0 = tc * G2::BN;
  const int k0 = split * kc, kn = min(kc, K - k0);
  C += (int64_t)split * M * N;
  const int lane = threadIdx.x & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
  G2RowsA ap;
  ap.c.init(A + k0, row0, M, K, w, lane);
  ap.w = w;
  G2Copy bc;
  bc.init(Bm + k0, col0, N, K, w, lane);
  f32x16 acc[2][4];
  g2_mainloop<true>(ap, bc, kn, As0, As1, Bs0, Bs1, acc);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = col0 + wn * 128 + nt * 32 + (lane & 31);
    if (col >= N) continue;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + g2_row(wm, mt, lane, r);
        if (row < M) C[row * N + col] = acc[mt][nt][r];
      }
  }
}

// Weight gradients C[M, N] = A^T B over the token dimension with both
// operands read in their own row-major layout, A [K, M] and B [K, N] (K = the
// token count): no transposed copies.  Tiles 256 x 256 x 64 on the forward's
// wave layout.  A 64-row slice of each operand (64 tokens x 256 columns, 512
// bytes per row) is copied straight into LDS with 16-byte chunk c of row r at
// c ^ 4 (r & 3), and the MFMA fragments are read with transposing LDS reads
// (ds_read_b64_tr_b16): lane l gets column 32 t + l % 32 at the eight k
// values kb + 4 (l / 32) + {0..3} and kb + 8 + 4 (l / 32) + {0..3}, the same
// k order for both operands, so every product pairs equal k.  Rows past K are
// clamped on load and zeroed in LDS before use; columns past M (N) clamp to the
// last full chunk and are never stored.  Split s covers rows
// [s * kc, min((s + 1) * kc, K)) and writes C + s * M * N.
typedef short tn_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tn_v4i16 tn_lds_v4i16;
struct TnCopy {
  static constexpr int PER = 4;  // 64 rows x 32 chunks / 512 threads
  int r[PER], cofs[PER];         // tile row and element column of each load
  __device__ __forceinline__ void init(int col0, int M, int w, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot = (w * PER + i) * 64 + lane;
      r[i] = slot >> 5;
      const int lc = (slot & 31) ^ (4 * (r[i] & 3));
      cofs[i] = min(col0 + lc * 8, M - 8);
    }
  }
  __device__ __forceinline__ void issue(const bf16* g, int64_t ld, int64_t k0, int64_t K, bf16* lds, int w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t t = min(k0 + r[i], K - 1);
      __builtin_amdgcn_global_load_lds((g2_glb_void*)(g + t * ld + cofs[i]),
                                       (g2_lds_void*)(lds + (w * PER + i) * 64 * 8), 16, 0, 0);
    }
  }
};
__device__ __forceinline__ bf16x8 tn_frag(const bf16* lds, int kb, int t, int lane) {
  const int a = lane & 15;
  const int row = kb + 4 * (lane >> 5) + (a >> 2);
  const int col = 32 * t + 16 * ((lane >> 4) & 1) + 4 * (a & 3);
  const int c = col >> 3, off = col & 7;
  const tn_v4i16 x0 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((tn_lds_v4i16*)(lds + row * 256 + ((c ^ (4 * (row & 3))) << 3) + off));
  const tn_v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (tn_lds_v4i16*)(lds + (row + 8) * 256 + ((c ^ (4 * ((row + 8) & 3))) << 3) + off));
  bf16x8 f;
  const bf16* p0 = reinterpret_cast<const bf16*>(&x0);
  const bf16* p1 = reinterpret_cast<const bf16*>(&x1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = p0[e];
    f[4 + e] = p1[e];
  }
  return f;
}

__global__ __launch_bounds__(512, 2) void gemm_tn_f32_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B,
                                                             float* __restrict__ C, int M, int N, int64_t K,
                                                             int64_t kc) {
  __shared__ __attribute__((aligned(16))) bf16 As0[64 * 256];
  __shared__ __attribute__((aligned(16))) bf16 As1[64 * 256];
  __shared__ __attribute__((aligned(16))) bf16 Bs0[64 * 256];
  __shared__ __attribute__((aligned(16))) bf16 Bs1[64 * 256];
  const int nrow = (M + 255) / 256, ncol = (N + 255) / 256;
  const int tiles = nrow * ncol, split = blockIdx.x / tiles;
  int tr, tc;
  map_tile(blockIdx.x - split * tiles, nrow, ncol, tr, tc);
  const int row0 = tr * 256, col0 = tc * 256;
  const int64_t kbeg = split * kc, kend = min(kbeg + kc, K);
  const int nk = (int)((kend - kbeg + 63) / 64);
  C += (int64_t)split * M * N;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
  TnCopy ac, bc;
  ac.init(row0, M, w, lane);
  bc.init(col0, N, w, lane);
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  // rows of the slice at k0 past kend read zero: clear them in this
  // thread's A chunks (its own copies, landed), before the barrier
  auto clear_tail = [&](int64_t k0, bf16* As) __attribute__((always_inline)) {
    if (k0 + 64 <= kend) return;  // workgroup-uniform
#pragma unroll
    for (int i = 0; i < TnCopy::PER; ++i)
      if (k0 + ac.r[i] >= kend)
        *reinterpret_cast<uint4*>(As + ((w * TnCopy::PER + i) * 64 + lane) * 8) = make_uint4(0, 0, 0, 0);
  };
  auto mma = [&](const bf16* As, const bf16* Bs) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[2], bfr[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) af[mt] = tn_frag(As, 16 * kk, wm * 2 + mt, lane);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bfr[nt] = tn_frag(Bs, 16 * kk, wn * 4 + nt, lane);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma_k16(af[mt], bfr[nt], acc[mt][nt]);
    }
  };
  // two slices per trip, each buffer a distinct LDS object; one barrier per slice
  if (nk > 0) {
    ac.issue(A, M, kbeg, K, As0, w);
    bc.issue(B, N, kbeg, K, Bs0, w);
  }
  int ks = 0;
  for (; ks + 2 <= nk; ks += 2) {
    const int64_t k0 = kbeg + (int64_t)ks * 64;
    __builtin_amdgcn_s_waitcnt(0);
    clear_tail(k0, As0);
    __syncthreads();
    ac.issue(A, M, k0 + 64, K, As1, w);
    bc.issue(B, N, k0 + 64, K, Bs1, w);
    mma(As0, Bs0);
    __builtin_amdgcn_s_waitcnt(0);
    clear_tail(k0 + 64, As1);
    __syncthreads();
    if (ks + 2 < nk) {
      ac.issue(A, M, k0 + 128, K, As0, w);
      bc.issue(B, N, k0 + 128, K, Bs0, w);
    }
    mma(As1, Bs1);
  }
  if (ks < nk) {  // odd slice count: the last slice is in buffer 0
    __builtin_amdgcn_s_waitcnt(0);
    clear_tail(kbeg + (int64_t)ks * 64, As0);
    __syncthreads();
    mma(As0, Bs0);
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = col0 + wn * 128 + nt * 32 + (lane & 31);
    if (col >= N) continue;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + g2_row(wm, mt, lane, r);
        if (row < M) C[(int64_t)row * N + col] = acc[mt][nt][r];
      }
  }
}

hipError_t launch_gemm_tn_f32(const void* A, const void* B, float* C, int M, int N, int64_t K, float* split_buf,
                              int64_t split_cap, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M % 8 != 0 || N % 8 != 0 || M < 8 || N < 8) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  // k splits: until the tiles give every compute unit one, chunks of at
  // least 1024 rows, and the partial products fit split_cap floats
  int S = 1;
  while (split_buf && S < 16 && tiles * S < 256 && K / (2 * S) >= 1024 && (int64_t)2 * S * M * N <= split_cap)
    S *= 2;
  const int64_t kc = ((K + S - 1) / S + 63) / 64 * 64;
  const int nsp = K > 0 ? (int)((K + kc - 1) / kc) : 1;
  float* out = nsp > 1 ? split_buf : C;
  hipLaunchKernelGGL(gemm_tn_f32_kernel, dim3((unsigned)(tiles * nsp)), dim3(512), 0, s, (const bf16*)A,
                     (const bf16*)B, out, M, N, K, kc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsp == 1) return e;
  const int64_t n = (int64_t)M * N;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)split_buf, n,
                     nsp, C);
  return hipGetLastError();
}

int gemm_splits(int64_t M, int N, int K) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int S = 1;
  while (S < kGemmMaxSplit && tiles * S < 512 && (int64_t)K / (2 * S) >= 512) S *= 2;
  return S;
}

// Splits for the 256 x 256 kernel: enough (sequence of k chunks, tile) work
// items to give every compute unit one, chunks of at least 1024.
static int gemm_splits_big(int64_t M, int N, int K) {
  const int64_t tiles = ((M + G2::BM - 1) / G2::BM) * ((N + G2::BN - 1) / G2::BN);
  int S = 1;
  while (S < kGemmMaxSplit && tiles * S < 256 && (int64_t)K / (2 * S) >= 1024) S *= 2;
  return S;
}

hipError_t launch_gemm_nt_f32(hstu_dtype dt, const void* A, const void* Bm, float* C, int64_t M, int N, int K,
                              float* split_buf, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (dt == HSTU_BF16 && K % G2::BK == 0) {
    const int64_t tiles = ((M + G2::BM - 1) / G2::BM) * ((N + G2::BN - 1) / G2::BN);
    const int S = split_buf ? gemm_splits_big(M, N, K) : 1;
    if (tiles * S >= 256) {
      const int kc = (int)((((int64_t)K + S - 1) / S + G2::BK - 1) / G2::BK * G2::BK);
      const int nsp = (int)((K + kc - 1) / kc);
      float* out = nsp > 1 ? split_buf : C;
      hipLaunchKernelGGL(gemm_nt_f32_big_kernel, dim3((unsigned)(tiles * nsp)), dim3(G2::NT), 0, s, (const bf16*)A,
                         (const bf16*)Bm, out, M, N, K, kc);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || nsp == 1) return e;
      const int64_t n = M * (int64_t)N;
      hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)split_buf,
                         n, nsp, C);
      return hipGetLastError();
    }
  }
  const int64_t nr = (M + 127) / 128, nc = (N + 127) / 128;
  const int S = split_buf ? gemm_splits(M, N, K) : 1;
  const int bk = dt == HSTU_BF16 ? 64 : 32;
  const int kc = (int)((((int64_t)K + S - 1) / S + bk - 1) / bk * bk);
  float* out = S > 1 ? split_buf : C;
  const dim3 grid((unsigned)(nr * nc * ((K + kc - 1) / kc)));
  if (dt == HSTU_BF16)
    hipLaunchKernelGGL(gemm_nt_f32_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)A, (const bf16*)Bm, out, M, N, K,
                       kc);
  else
    hipLaunchKernelGGL(gemm_nt_f32_kernel<float>, grid, dim3(256), 0, s, (const float*)A, (const float*)Bm, out, M,
                       N, K, kc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t n = M * (int64_t)N;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)split_buf, n,
                     (int)((K + kc - 1) / kc), C);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const hstu_desc& d, int64_t T, const hstu_weights& w, const float* dz, const void* u,
                           const void* av, const float* stats, const void* pre, void* dpre, void* dav, float* gpart,
                           float* bpart, float* dg, float* db, hipStream_t s) {
  const int K = d.num_heads * d.dv;
  if (K % 8 != 0 || K > kBwdRowCols) return hipErrorInvalidValue;
  const int64_t n1 = 2 * (int64_t)d.num_heads * (d.dqk + d.dv);
  const int64_t chunks = (T + kChunkRows - 1) / kChunkRows;
  if (chunks > 0) {
    const dim3 grid((unsigned)chunks), block(256);
    const size_t shmem = (size_t)8 * K * sizeof(float);
    with_chunks(K, [&](auto nc) {
      constexpr int NC = decltype(nc)::value;
      if (d.dtype == HSTU_BF16)
        hipLaunchKernelGGL((gate_bwd_kernel<bf16, NC>), grid, block, shmem, s, dz, (const bf16*)u, (const bf16*)av,
                           stats, (const bf16*)w.ln_av_g, (const bf16*)w.ln_av_b, T, d.num_heads, d.dv, d.ln_eps, n1,
                           (const bf16*)pre, (bf16*)dpre, (bf16*)dav, gpart, bpart);
      else
        hipLaunchKernelGGL((gate_bwd_kernel<float, NC>), grid, block, shmem, s, dz, (const float*)u, (const float*)av,
                           stats, (const float*)w.ln_av_g, (const float*)w.ln_av_b, T, d.num_heads, d.dv, d.ln_eps,
                           n1, (const float*)pre, (float*)dpre, (float*)dav, gpart, bpart);
    });
  }
  const dim3 cg((unsigned)((K + 63) / 64)), cb(64 * kColGroups);
  hipLaunchKernelGGL(colsum_chunks_kernel, cg, cb, 0, s, (const float*)gpart, chunks, (int64_t)K, dg);
  hipLaunchKernelGGL(colsum_chunks_kernel, cg, cb, 0, s, (const float*)bpart, chunks, (int64_t)K, db);
  return hipGetLastError();
}


hipError_t launch_ln_bwd(const hstu_desc& d, const void* x, const float* dxn, const hstu_weights& w, const void* dy,
                         int64_t T, void* dx, float* gpart, float* bpart, float* dg, float* db, hipStream_t s) {
  const int dm = d.d_model;
  if (dm % 8 != 0 || dm > kBwdRowCols) return hipErrorInvalidValue;
  const int norm = (d.flags & HSTU_INPUT_NORM) ? 1 : 0, res = (d.flags & HSTU_RESIDUAL) ? 1 : 0;
  const int64_t chunks = (T + kChunkRows - 1) / kChunkRows;
  if (chunks > 0) {
    const dim3 grid((unsigned)chunks), block(256);
    const size_t shmem = (size_t)8 * dm * sizeof(float);
    with_chunks(dm, [&](auto nc) {
      constexpr int NC = decltype(nc)::value;
      if (d.dtype == HSTU_BF16)
        hipLaunchKernelGGL((ln_bwd_kernel<bf16, NC>), grid, block, shmem, s, (const bf16*)x, dxn,
                           (const bf16*)w.ln_in_g, (const bf16*)dy, T, dm, d.ln_eps, norm, res, (bf16*)dx, gpart,
                           bpart);
      else
        hipLaunchKernelGGL((ln_bwd_kernel<float, NC>), grid, block, shmem, s, (const float*)x, dxn,
                           (const float*)w.ln_in_g, (const float*)dy, T, dm, d.ln_eps, norm, res, (float*)dx, gpart,
                           bpart);
    });
  }
  // without the input LayerNorm its parameters get zero gradients
  const dim3 cg((unsigned)((dm + 63) / 64)), cb(64 * kColGroups);
  hipLaunchKernelGGL(colsum_chunks_kernel, cg, cb, 0, s, (const float*)gpart, norm ? chunks : 0, (int64_t)dm, dg);
  hipLaunchKernelGGL(colsum_chunks_kernel, cg, cb, 0, s, (const float*)bpart, norm ? chunks : 0, (int64_t)dm, db);
  return hipGetLastError();
}

}  // namespace hstu
