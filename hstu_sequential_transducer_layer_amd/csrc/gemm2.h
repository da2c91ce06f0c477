// Large-tile "NT" GEMM core for bf16: C[M, N] = A[M, K] * B[N, K]^T, both
// operands K-contiguous, K a multiple of 64.
//
// Tile 256 x 256 x 64 on 512 threads (8 waves in 4 x 2, each wave 64 x 128 =
// 2 x 4 MFMA 32x32x16 tiles, 128 fp32 accumulators per lane; one workgroup
// per CU, two waves per SIMD).  B rows — and A rows when A is a plain matrix — are copied global->LDS
// with 16-byte direct loads into two buffers (the copy of step k+1 runs while
// step k is multiplied).  An A operand that is a function of several inputs
// (LayerNorm + gate) is produced through registers, one 16-byte chunk per
// (row, 8 columns) per workgroup, and stored into the same LDS layout.
// LDS rows are 128 bytes = 8 chunks; chunk c of row r lives at
// c ^ ((r >> 1) & 7): the LDS has 64 four-byte banks (256 bytes), so a 16-byte
// read by 16 lanes of 16 consecutive rows covers every bank once.
#pragma once

#include "common.h"

namespace hstu {

typedef __attribute__((address_space(3))) void g2_lds_void;
typedef __attribute__((address_space(1))) void g2_glb_void;

// Below this many 256 x 256 tiles a projection launch leaves most compute
// units idle, and the 128 x 128 kernel (four times the tiles) finishes first
// (measured on a 2048-row candidate micro-batch: 16 us against 21 us).  The
// f2 GEMM keeps the large tiles at every size: its 128 x 128 kernel was
// slower even there.
constexpr int64_t kG2MinTiles = 128;

struct G2 {
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int NT = 512;            // threads
  static constexpr int WM = 4, WN = 2;      // wave grid
  static constexpr int TM = 2, TN = 4;      // MFMA tiles per wave (rows, cols)
  static constexpr int CPR = BK / 8;        // 16-byte chunks per tile row
  static constexpr int A_CH = BM * CPR;     // chunks per A stage (2048)
  static constexpr int B_CH = BN * CPR;
  static constexpr int STAGE = BM * BK;     // elements per A (or B) stage
};

__device__ __forceinline__ int g2_swz(int r) { return (r >> 1) & 7; }

// Direct copies of a 256-row x 64-column bf16 tile of a [rows, K] matrix into
// an LDS stage.  Each thread issues PER 16-byte loads; their per-lane element
// offsets (row * K + chunk * 8, relative to the tile's first row) are fixed for
// the whole K loop and computed once.  Rows past `rows` re-read the last row
// (their products land in outputs that are never stored).
struct G2Copy {
  static constexpr int PER = G2::A_CH / G2::NT;  // 4 loads per thread per stage
  const bf16* base;                             // first element of the tile's first row
  int off[PER];
  __device__ __forceinline__ void init(const bf16* g, int64_t row0, int64_t rows, int K, int w, int lane) {
    base = g + row0 * K;
    const int64_t last = rows - 1 - row0;  // last valid tile row
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot = (w * PER + i) * 64 + lane;
      const int r = slot / G2::CPR, pc = slot % G2::CPR;
      const int rr = r <= last ? r : (int)last;
      off[i] = rr * K + ((pc ^ g2_swz(r)) * 8);
    }
  }
  __device__ __forceinline__ void issue(int k0, bf16* lds, int w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int slot0 = (w * PER + i) * 64;
      __builtin_amdgcn_global_load_lds((g2_glb_void*)(base + k0 + off[i]), (g2_lds_void*)(lds + slot0 * 8),
                                       16, 0, 0);
    }
  }
};

// 16-byte chunk store into the swizzled layout (register-produced A operand).
__device__ __forceinline__ void g2_store_chunk(bf16* lds, int r, int c, const uint4& v) {
  *reinterpret_cast<uint4*>(lds + r * G2::BK + ((c ^ g2_swz(r)) * 8)) = v;
}

__device__ __forceinline__ bf16x8 g2_frag(const bf16* lds, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(lds + r * G2::BK + ((c ^ g2_swz(r)) * 8));
}

// The MFMAs of one 64-wide K step for one wave.  With PIPE the operands of
// k16 step kk + 1 are read while step kk's MFMAs run (two fragment sets live);
// without it one set is live, for callers that hold other data in registers.
template <bool PIPE>
__device__ __forceinline__ void g2_mma_step(const bf16* As, const bf16* Bs, f32x16 (&acc)[2][4],
                                            int wm, int wn, int lane) {
  const int l32 = lane & 31, half = lane >> 5;
  constexpr int NB = PIPE ? 2 : 1;
  bf16x8 af[NB][2], bfr[NB][4];
  auto load = [&](int kk, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) af[buf][t] = g2_frag(As, wm * 64 + t * 32 + l32, 2 * kk + half);
#pragma unroll
    for (int t = 0; t < 4; ++t) bfr[buf][t] = g2_frag(Bs, wn * 128 + t * 32 + l32, 2 * kk + half);
  };
  if (PIPE) load(0, 0);
#pragma unroll
  for (int kk = 0; kk < G2::BK / 16; ++kk) {
    const int cur = PIPE ? (kk & 1) : 0;
    if (PIPE) {
      if (kk + 1 < G2::BK / 16) load(kk + 1, cur ^ 1);
    } else {
      load(kk, 0);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mma_k16(af[cur][mt], bfr[cur][nt], acc[mt][nt]);
  }
}

// Row within the block tile of accumulator element r of wave tile (wm, mt).
__device__ __forceinline__ int g2_row(int wm, int mt, int lane, int r) {
  return wm * 64 + mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Main loop.  AProd::start(k0, buf) begins producing A stage `buf` for the
// K step at k0 (direct copies are asynchronous; register producers load now
// and store in finish()); AProd::finish(buf) completes it before the barrier.
// Two K steps per trip so each LDS buffer is a distinct object (the compiler
// then needs no wait on the in-flight copy before reading the other buffer).
template <bool PIPE, class AProd>
__device__ __forceinline__ void g2_mainloop(AProd& ap, const G2Copy& bc, int K, bf16* As0, bf16* As1,
                                            bf16* Bs0, bf16* Bs1, f32x16 (&acc)[2][4]) {
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  const int nk = K / G2::BK;
  ap.start(0, As0);
  bc.issue(0, Bs0, w);
  ap.finish(As0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int ks = 0;
  for (; ks + 2 <= nk; ks += 2) {
    ap.start((ks + 1) * G2::BK, As1);
    bc.issue((ks + 1) * G2::BK, Bs1, w);
    g2_mma_step<PIPE>(As0, Bs0, acc, wm, wn, lane);
    ap.finish(As1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool more = ks + 2 < nk;
    if (more) {
      ap.start((ks + 2) * G2::BK, As0);
      bc.issue((ks + 2) * G2::BK, Bs0, w);
    }
    g2_mma_step<PIPE>(As1, Bs1, acc, wm, wn, lane);
    if (more) {
      ap.finish(As0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
  if (ks < nk) g2_mma_step<PIPE>(As0, Bs0, acc, wm, wn, lane);  // odd step count: last stage is in buffer 0
}

// ---------------------------------------------------------------- epilogue
// The 256 x 256 output tile is staged through LDS so that global loads and
// stores move 16 bytes per lane along rows: 64-row quarter q of the tile lives
// in operand stage q (32 KB each), row-major, with 16-byte chunk c of row r at
// chunk c ^ g2_out_swz(r).  In the accumulator phase a wave touches 32
// consecutive columns of rows R and R + 4 (2 bytes per lane); the swizzle puts
// those two rows on different banks.  In the row phase, "slot" s = i * 512 +
// tid (i = 0..15) is row s / 32, physical chunk s % 32 of the tile, so each
// thread keeps one logical column chunk for all its rows.
__device__ __forceinline__ int g2_out_swz(int r) { return ((r >> 2) & 1) << 2; }

// Element offset of (row within quarter, column within tile).
__device__ __forceinline__ int g2_out_off(int r, int col) {
  return r * G2::BN + (((col >> 3) ^ g2_out_swz(r)) << 3) + (col & 7);
}

// Row within the quarter of accumulator element r of wave tile (wm, mt).
__device__ __forceinline__ int g2_out_row(int mt, int lane, int r) {
  return mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Logical column chunk of this thread in the row phase.
__device__ __forceinline__ int g2_out_chunk(int tid) { return (tid & 31) ^ g2_out_swz(tid >> 5); }

// Row phase: copy rows [row0, row0 + 256) x columns [col0, col0 + 256) of a
// [M, ld] bf16 matrix into the staged tile (direct global->LDS, 16 bytes per
// lane).  Rows past M and column chunks past N read valid elements instead;
// those tile entries are never stored.
struct G2Quarters {
  bf16 *q0, *q1, *q2, *q3;
  __device__ __forceinline__ bf16* operator[](int i) const { return i == 0 ? q0 : i == 1 ? q1 : i == 2 ? q2 : q3; }
};

__device__ __forceinline__ void g2_out_load(const bf16* g, int64_t row0, int64_t M, int col0, int N, int ld,
                                            const G2Quarters& qs, int tid, int w) {
  const int col = col0 + 8 * g2_out_chunk(tid);
  const int colc = col < N ? col : 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int R = (i * G2::NT + tid) >> 5;
    const int64_t row = row0 + R < M ? row0 + R : M - 1;
    __builtin_amdgcn_global_load_lds((g2_glb_void*)(g + row * ld + colc),
                                     (g2_lds_void*)(qs[i >> 2] + ((i & 3) * G2::NT + w * 64) * 8), 16, 0, 0);
  }
}

// A operand = plain rows of a [M, K] matrix, copied directly.
struct G2RowsA {
  G2Copy c;
  int w;
  __device__ __forceinline__ void start(int k0, bf16* lds) { c.issue(k0, lds, w); }
  __device__ __forceinline__ void finish(bf16*) {}
};

}  // namespace hstu
