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
#include "common.h"
#include "gemm.h"
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

// One wave per row.  Recomputes the LayerNorm of AV from the attention's
// per-head statistics (the forward gate's merge), then
//   n^ = (AV - mean) * rstd,  dn = dZ * U,  dn^ = dn * g
//   dU = dZ * (n^ g + b),  dAV = rstd (dn^ - mean(dn^) - n^ mean(dn^ n^))
// and the per-row terms dn * n^ and dn of dg and db.
template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float* __restrict__ dz, const T* __restrict__ u,
                                                       const T* __restrict__ av, const float* __restrict__ stats,
                                                       const T* __restrict__ g, const T* __restrict__ be,
                                                       int64_t M, int H, int dv, float eps, int64_t n1,
                                                       float* __restrict__ du, T* __restrict__ dav,
                                                       float* __restrict__ gterm, float* __restrict__ bterm) {
  // one wave per row; a lane takes 8 consecutive columns of one head per step
  // (dv a multiple of 8)
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= M) return;
  const int K = H * dv;
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
  for (int c = lane * 8; c < K; c += 8 * kWave) {
    const float off = __shfl(dm, c / dv, kWave);
    float b8[8], o_du[8], o_dav[8], o_g[8], o_b[8];
    load8(av + o + c, a8);
    load8(dz + o + c, z8);
    load8(u + o + c, u8);
    load8(g + c, g8);
    load8(be + c, b8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float nh = (a8[e] + off) * rstd;
      const float dn = z8[e] * u8[e];
      o_du[e] = z8[e] * (nh * g8[e] + b8[e]);
      o_dav[e] = rstd * (dn * g8[e] - m1 - nh * mm);
      o_g[e] = dn * nh;
      o_b[e] = dn;
    }
    store8(du + row * n1 + c, o_du);
    store8(dav + o + c, o_dav);
    store8(gterm + o + c, o_g);
    store8(bterm + o + c, o_b);
  }
}

// The pre-activation GEMM of f1 with the SiLU backward as its epilogue: the
// 128 x 128 tile pre = A B^T (A = x~ [M, K], B = W1 [N, K]) never leaves the
// chip.  z = pre + b1 goes through LDS, 64 rows at a time (rows padded to 136
// floats, so the accumulator writes of a wave's two 4-row groups hit
// different banks), and is read back along rows: each thread takes 8 columns
// of one row per pass, loads dact with 16-byte loads and writes dpre =
// dact * SiLU'(z) in the layer dtype.  The tile's 128 rows are one row chunk
// of db1's column sums: a thread adds its rows in order, then the 16 row
// groups are added in order into part[chunk][col].  N is a multiple of 8.
constexpr int kSiluPad = 136;
template <typename T>
__global__ __launch_bounds__(256, 2) void gemm_silu_bwd_kernel(const T* __restrict__ A, const T* __restrict__ Bm,
                                                               const T* __restrict__ b1, const float* __restrict__ dact,
                                                               int64_t M, int N, int K, T* __restrict__ dpre,
                                                               float* __restrict__ part) {
  typedef GemmTile<T> G;
  static_assert(G::BM == kColRows && G::BM == 128 && G::BN == 128, "a tile row is one row chunk of the column sums");
  __shared__ __attribute__((aligned(16))) T As[G::BM * G::LDK];
  __shared__ __attribute__((aligned(16))) T Bs[G::BN * G::LDK];
  __shared__ __attribute__((aligned(16))) float zs[64 * kSiluPad];
  __shared__ float red[16][G::BN];
  const int nrow = (int)((M + G::BM - 1) / G::BM), ncol = (N + G::BN - 1) / G::BN;
  int tr, tc;
  map_tile(blockIdx.x, nrow, ncol, tr, tc);
  const int64_t row0 = (int64_t)tr * G::BM;
  const int col0 = tc * G::BN;
  RowLoader<T> al{A, row0, M, K, K};
  f32x16 acc[2][2];
  gemm_mainloop<T>(al, Bm, col0, N, K, As, Bs, acc, K);
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), wm = w >> 1, wn = w & 1;
  float bias[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int col = col0 + wn * 64 + nt * 32 + (lane & 31);
    bias[nt] = col < N ? to_f32(b1[col]) : 0.f;
  }
  const int rr = tid >> 4, cg = tid & 15;  // read phase: row group, 8-column group
  const int gcol = col0 + cg * 8;
  float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    if (wm == hf) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            zs[(acc_row(0, mt, lane, r)) * kSiluPad + wn * 64 + nt * 32 + (lane & 31)] = acc[mt][nt][r] + bias[nt];
    }
    __syncthreads();
#pragma unroll
    for (int pss = 0; pss < 4; ++pss) {
      const int lr = pss * 16 + rr;
      const int64_t grow = row0 + hf * 64 + lr;
      if (grow < M && gcol < N) {
        const float4 z0 = *reinterpret_cast<const float4*>(zs + lr * kSiluPad + cg * 8);
        const float4 z1 = *reinterpret_cast<const float4*>(zs + lr * kSiluPad + cg * 8 + 4);
        const float* gp = dact + grow * N + gcol;
        const float4 g0 = *reinterpret_cast<const float4*>(gp), g1 = *reinterpret_cast<const float4*>(gp + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        T out[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float z = zv[q];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
          const float d = gv[q] * sg * (1.0f + z * (1.0f - sg));
          cs[q] += d;
          out[q] = from_f32<T>(d);
        }
        T* dst = dpre + grow * N + gcol;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(out);
        } else {
          *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(out);
          *reinterpret_cast<float4*>(dst + 4) = *reinterpret_cast<const float4*>(out + 4);
        }
      }
    }
    __syncthreads();  // zs is rewritten by the next half
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) red[rr][cg * 8 + q] = cs[q];
  __syncthreads();
  if (tid < G::BN && col0 + tid < N) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) sum += red[g][tid];
    part[(int64_t)tr * N + col0 + tid] = sum;
  }
}

// One wave per row.  With the input LayerNorm: x^ = (x - mean) rstd,
// dx = rstd (dxn g - mean(dxn g) - x^ mean(dxn g x^)); else dx = dxn.  Plus dY
// for the residual.  gterm = dxn * x^ (per-row term of the gain's gradient).
template <typename T>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const T* __restrict__ x, const float* __restrict__ dxn,
                                                     const T* __restrict__ g, const T* __restrict__ dy, int64_t M,
                                                     int d, float eps, int norm, int residual, T* __restrict__ dx,
                                                     float* __restrict__ gterm) {
  // one wave per row; a lane takes 8 consecutive columns per step (16-byte
  // accesses for bf16), d a multiple of 8
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  if (row >= M) return;
  const int64_t o = row * d;
  float mean = 0.f, rstd = 1.f, m1 = 0.f, mm = 0.f;
  float xv[8], gv[8], dv8[8];
  if (norm) {
    float s = 0.f;
    for (int c = lane * 8; c < d; c += 8 * kWave) {
      load8(x + o + c, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += xv[e];
    }
    mean = wave_sum(s) / (float)d;
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
  for (int c = lane * 8; c < d; c += 8 * kWave) {
    float r[8], gt[8], yv[8];
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
        gt[e] = dv8[e] * xh;
      } else {
        r[e] = dv8[e];
      }
      if (residual) r[e] += yv[e];
    }
    if (norm) store8(gterm + o + c, gt);
    store8(dx + o + c, r);
  }
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

int gemm_splits(int64_t M, int N, int K) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int S = 1;
  while (S < kGemmMaxSplit && tiles * S < 512 && (int64_t)K / (2 * S) >= 512) S *= 2;
  return S;
}

hipError_t launch_gemm_nt_f32(hstu_dtype dt, const void* A, const void* Bm, float* C, int64_t M, int N, int K,
                              float* split_buf, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
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
                           const void* av, const float* stats, float* du, void* dav, float* gterm, float* bterm,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t n1 = 2 * (int64_t)d.num_heads * (d.dqk + d.dv);
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL(gate_bwd_kernel<bf16>, grid, block, 0, s, dz, (const bf16*)u, (const bf16*)av, stats,
                       (const bf16*)w.ln_av_g, (const bf16*)w.ln_av_b, T, d.num_heads, d.dv, d.ln_eps, n1, du,
                       (bf16*)dav, gterm, bterm);
  else
    hipLaunchKernelGGL(gate_bwd_kernel<float>, grid, block, 0, s, dz, (const float*)u, (const float*)av, stats,
                       (const float*)w.ln_av_g, (const float*)w.ln_av_b, T, d.num_heads, d.dv, d.ln_eps, n1, du,
                       (float*)dav, gterm, bterm);
  return hipGetLastError();
}

hipError_t launch_gemm_silu_bwd(hstu_dtype dt, const void* A, const void* w1, const void* b1, const float* dact,
                                int64_t T, int n1, int K, void* dpre_t, float* part, float* db1, hipStream_t s) {
  if (n1 % 8 != 0 || K % 8 != 0) return hipErrorInvalidValue;
  const int64_t chunks = (T + kColRows - 1) / kColRows;
  if (chunks > 0) {
    const dim3 grid((unsigned)(chunks * ((n1 + 127) / 128)));
    if (dt == HSTU_BF16)
      hipLaunchKernelGGL(gemm_silu_bwd_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)A, (const bf16*)w1,
                         (const bf16*)b1, dact, T, n1, K, (bf16*)dpre_t, part);
    else
      hipLaunchKernelGGL(gemm_silu_bwd_kernel<float>, grid, dim3(256), 0, s, (const float*)A, (const float*)w1,
                         (const float*)b1, dact, T, n1, K, (float*)dpre_t, part);
  }
  hipLaunchKernelGGL(colsum_chunks_kernel, dim3((unsigned)((n1 + 63) / 64)), dim3(64 * kColGroups), 0, s,
                     (const float*)part, chunks, (int64_t)n1, db1);
  return hipGetLastError();
}

hipError_t launch_ln_bwd(const hstu_desc& d, const void* x, const float* dxn, const hstu_weights& w, const void* dy,
                         int64_t T, void* dx, float* gterm, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int norm = (d.flags & HSTU_INPUT_NORM) ? 1 : 0, res = (d.flags & HSTU_RESIDUAL) ? 1 : 0;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL(ln_bwd_kernel<bf16>, grid, block, 0, s, (const bf16*)x, dxn, (const bf16*)w.ln_in_g,
                       (const bf16*)dy, T, d.d_model, d.ln_eps, norm, res, (bf16*)dx, gterm);
  else
    hipLaunchKernelGGL(ln_bwd_kernel<float>, grid, block, 0, s, (const float*)x, dxn, (const float*)w.ln_in_g,
                       (const float*)dy, T, d.d_model, d.ln_eps, norm, res, (float*)dx, gterm);
  return hipGetLastError();
}

}  // namespace hstu
