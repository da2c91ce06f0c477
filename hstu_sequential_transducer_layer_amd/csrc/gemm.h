// Tiled "NT" GEMM skeleton on MFMA: C[M, N] = A[M, K] * B[N, K]^T with both
// operands K-contiguous (nn.Linear weight layout).  The A operand is produced
// by a caller-supplied functor (plain rows for f1, LayerNorm+gate for f2), the
// epilogue is the caller's.
//
// Tile 128 x 128 x (128 bytes of K), 256 threads = 4 waves in a 2 x 2 grid, each wave owning
// 64 x 64 = 2 x 2 MFMA 32x32 tiles.  Global loads for step k+1 are issued
// before the MFMAs of step k and parked in registers (one LDS buffer).
// LDS rows are padded by 16 bytes so the 16-byte operand reads of 8
// consecutive rows fall in distinct banks.
#pragma once

#include "common.h"

namespace hstu {

template <typename T>
struct GemmTile {
  static constexpr int BM = 128, BN = 128;
  static constexpr int BK = 128 / (int)sizeof(T);       // 128-byte tile rows (64 bf16)
  static constexpr int V = Elem<T>::kVec;
  static constexpr int LDK = BK + 16 / (int)sizeof(T);
  static constexpr int CPR = BK / V;                    // 16-byte chunks per tile row
  static constexpr int NCH = BM * CPR / 256;            // chunks per thread per operand
};

// Block id -> (row tile, column tile).  Workgroups are dispatched round-robin
// over the 8 XCDs, so ids x, x+8, x+16, ... share XCD x's L2: give each XCD a
// contiguous range of tiles, and walk that range in groups of kGroupRows row
// tiles (column-major inside a group) so co-resident workgroups share both
// the A rows and the B rows they stream.
constexpr int kXcds = 8;
constexpr int kGroupRows = 8;

__device__ __forceinline__ void map_tile(int bid, int nrow, int ncol, int& tr, int& tc) {
  const int n = nrow * ncol;
  const int xcd = bid % kXcds, local = bid / kXcds;
  // XCD x receives ids x, x+8, ...: ceil((n - x) / 8) of them.
  const int base = n / kXcds, extra = n % kXcds;
  const int tile = xcd * base + min(xcd, extra) + local;
  const int gsize = kGroupRows * ncol;
  const int g = tile / gsize, in = tile % gsize;
  const int r0 = g * kGroupRows;
  const int rows = min(kGroupRows, nrow - r0);
  tr = r0 + in % rows;
  tc = in / rows;
}

// A operand = plain rows of a [M, K] matrix.
template <typename T>
struct RowLoader {
  const T* __restrict__ a;
  int64_t row0, M;
  int K;
  int64_t ld = 0;  // row stride when it is not K (a column slice of a wider matrix)
  __device__ __forceinline__ uint4 operator()(int k0, int r, int kc) const {
    const int64_t row = row0 + r;
    const int k = k0 + kc;
    return (row < M && k < K) ? ld16(a + row * (ld ? ld : (int64_t)K) + k) : make_uint4(0, 0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag lds_frag(const T* p) {
  return *reinterpret_cast<const typename Elem<T>::Frag*>(p);
}

// Main loop.  `aload(chunk, k0, r, kc)` returns the 16-byte A chunk for tile
// row r, columns k0+kc .. k0+kc+V-1 (zero outside the matrix).  B rows come
// from `b` [N, K].  acc[mt][nt] holds the wave's 2 x 2 MFMA tiles.
template <typename T, class ALoad>
__device__ __forceinline__ void gemm_mainloop(ALoad& aload, const T* __restrict__ b, int64_t col0,
                                              int N, int K, T* As, T* Bs, f32x16 (&acc)[2][2], int64_t ldb = 0) {
  typedef GemmTile<T> G;
  const int64_t bstride = ldb ? ldb : (int64_t)K;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int wm = w >> 1, wn = w & 1;
  uint4 ra[G::NCH], rb[G::NCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int c = 0; c < G::NCH; ++c) {
      const int idx = tid + c * 256;
      const int r = idx / G::CPR, kc = (idx % G::CPR) * G::V;
      ra[c] = aload(k0, r, kc);
      const int64_t n = col0 + r;
      const int k = k0 + kc;
      rb[c] = (n < N && k < K) ? ld16(b + n * bstride + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int c = 0; c < G::NCH; ++c) {
      const int idx = tid + c * 256;
      const int r = idx / G::CPR, kc = (idx % G::CPR) * G::V;
      st16(As + r * G::LDK + kc, ra[c]);
      st16(Bs + r * G::LDK + kc, rb[c]);
    }
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  gload(0);
  for (int k0 = 0; k0 < K; k0 += G::BK) {
    sstore();
    __syncthreads();
    if (k0 + G::BK < K) gload(k0 + G::BK);
#pragma unroll
    for (int kk = 0; kk < G::BK / 16; ++kk) {
      const int ko = kk * 16 + 8 * (lane >> 5);
      typename Elem<T>::Frag af[2], bf[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) af[mt] = lds_frag(As + (wm * 64 + mt * 32 + (lane & 31)) * G::LDK + ko);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bf[nt] = lds_frag(Bs + (wn * 64 + nt * 32 + (lane & 31)) * G::LDK + ko);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma_k16(af[mt], bf[nt], acc[mt][nt]);
    }
    __syncthreads();
  }
}

// Row of output element r of a wave's MFMA tile (mt) within the block tile.
__device__ __forceinline__ int acc_row(int wm, int mt, int lane, int r) {
  return wm * 64 + mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

}  // namespace hstu
