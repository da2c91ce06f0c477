// Backward of the pointwise attention — the gradient of
//   AV_i^h = sum_j a_ij v_j,   a_ij = M_ij SiLU(S_ij) / N_b,
//   S_ij = q_i.k_j + pos[h][bp(i,j)] + time[h][bt(i,j)]
// (page "4.4 Scaling Recommendation Models", section "Generative Recommenders
// and HSTU", second layer equation and its bullets, and section "Code"; page
// "HSTU: The First Exploration of the Scaling Law", 7.1.4 Innovations 1-2 and
// 7.1.5 M-FALCON mask).  With dO = dL/dAV:
//   dv_j = sum_i a_ij dO_i                 dS_ij = (dO_i.v_j) M_ij SiLU'(S_ij) / N_b
//   dq_i = sum_j dS_ij k_j                 dk_j  = sum_i dS_ij q_i
//   dpos[h][b] = sum over pairs with bp = b of dS_ij, dtime likewise.
// Pointwise weights need no softmax statistics: S is recomputed per tile.
//
// attn_bwd_dq_kernel: work item (sequence, 128-row query tile, head), the
//   forward's work list; the key blocks of the forward.  Per 32-key half:
//   S^T = K Q^T and dA^T = V dO^T on MFMA (K, V rows from LDS, Q, dO in
//   registers), dS^T in registers, dQ^T += K^T dS^T (K^T read element-wise
//   from LDS, dS^T straight from the accumulators as the B operand).  The
//   bias-table gradients gather in LDS histograms, one row of partial sums
//   per workgroup.
// attn_bwd_dkv_kernel<DK>: work item (sequence, 128-key tile, head); every
//   query block that can see those keys.  S = Q K^T (Q rows from LDS, K in
//   registers); DK = false: dV^T += dO^T a; DK = true: dA = dO V^T and
//   dK^T += Q^T dS.  Two passes keep each pass's accumulators in registers.
// attn_bwd_kv16_kernel (bf16): dK and dV in one pass (described there).
// PRE kernels write each gradient times SiLU'(pre), the forward's saved
// pre-activation, straight into the layer backward's dpre; the others write
// the raw gradients in fp32.
// K/V (Q/dO) blocks are staged in LDS by direct global->LDS loads, double
// buffered: block b + 1 is copied while block b is consumed.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hstu {

struct BwdArgs {
  const int64_t* off;
  const int32_t* ncand;
  const int64_t* ts;
  const void* pos_tab;
  const void* time_tab;
  const void* q;      // [H, T, DQK]
  const void* k;      // [H, T, DQK]
  const void* v;      // [H, T, DV]
  const void* dout;   // [T, H * DV]: dL/dAV
  float* dact;        // [T, N1]: dv at column K2 + h DV, dq at 2 K2 + h DQK, dk at 2 K2 + H DQK + h DQK
  const void* pre;    // PRE kernels: the saved pre-activation [T, N1] (layer dtype) ...
  void* dpre;         // ... and the gradients times SiLU'(pre) in its layout, in place of dact
  float* tab_part;    // [gridDim.x][P + NB]: per-workgroup bias-table gradients (dq kernel),
                      // row (tbase[b] + query tile) * H + h: fixed by the batch, not by
                      // where the item sits in the work list
  const int2* tiles;
  const int32_t* tbase;  // first query tile of each sequence
  const int32_t* counts;
  const int64_t* tstat;  // per 64-row block's first row: its earliest, latest timestamp
  int64_t T;
  int H, P, NB, sbits, pos_stride, time_stride, norm_len, shared_pos, N1;
};

typedef __attribute__((address_space(3))) void bwd_lds_void;
typedef __attribute__((address_space(1))) void bwd_glb_void;

// Tiles in LDS: 64 rows of D elements, row-major without padding; chunk c
// (one 16-byte vector of kVec elements) of row r is stored at chunk
// c ^ bwd_swz(r).  The swizzle spreads both access patterns over the banks:
// 16 consecutive rows read 16 bytes each at one logical chunk (row
// fragments), and four consecutive rows read as two adjacent chunks each (the
// transposing reads of column fragments).  For 16-chunk rows the swizzle was
// chosen by timing both patterns on the hardware against alternatives (the
// earlier one cost the dq kernel 4.8% of its cycles in bank conflicts).
// bwd_swz(0) = 0 and bwd_swz depends on r % 16 only.
template <int CPR>
__device__ __forceinline__ int bwd_swz(int r) {
  if constexpr (CPR >= 16) {
    return (4 * (r & 3)) ^ ((r >> 2) & 3);
  } else if constexpr (CPR == 8) {
    const int x = r >> 1;
    return ((x & 1) << 1) | ((x >> 1) & 1) | (x & 4);
  } else {
    return (r >> 2) & 3;
  }
}

template <typename T, int D>
struct BTile {
  static constexpr int V = Elem<T>::kVec, CPR = D / V;
  static_assert(CPR >= 4 && CPR <= 16, "tile width");
  // element offset of element e of row r
  static __device__ __forceinline__ int at(int r, int e) { return r * D + (((e / V) ^ bwd_swz<CPR>(r)) * V) + e % V; }
};

// The merged dK/dV kernel's bf16 tiles (16 x 16 MFMA fragments) read them in
// two other patterns: 16 consecutive rows at one logical chunk (row
// fragments), and eight consecutive rows at two adjacent chunks per 32 lanes
// (transposing reads).  With 64 four-byte banks both are free of conflicts
// when, over any 16 rows, the rows that share a bank window get distinct
// physical chunks and, over any aligned 8 rows, kv_swz(r) >> 1 takes distinct
// values (checked exhaustively on the host).  Depends on r % 16 only.
template <int CPR>
__device__ __forceinline__ int kv_swz(int r) {
  constexpr int SH = CPR >= 16 ? 0 : (CPR == 8 ? 1 : 2);
  return (((r & 7) >> SH) << 1) | ((r >> 3) & 1);
}

template <int D>
struct KvTile {
  static constexpr int CPR = D / 8;
  static_assert(CPR >= 4 && CPR <= 16, "tile width");
  static __device__ __forceinline__ int at(int r, int e) { return r * D + (((e >> 3) ^ kv_swz<CPR>(r)) << 3) + (e & 7); }
};

// Asynchronous copy of 64 rows (row stride S elements in global memory) into a
// swizzled tile by direct global->LDS loads: each of the four waves issues PER
// 16-byte-per-lane loads; load i of wave w fills the 64 / CPR rows from
// (4 i + w) * 64 / CPR, so a lane's rows lie STRIDE (a multiple of 16) rows
// apart and share one swizzle.  Rows at or past `avail` (>= 1) repeat row
// avail - 1.  KV selects kv_swz (KvTile) in place of bwd_swz (BTile).
template <typename T, int D, bool KV = false>
struct BwdCopy {
  static constexpr int V = Elem<T>::kVec, CPR = D / V, PER = CPR / 4, STRIDE = 256 / CPR;
  static_assert(PER == 1 || STRIDE % 16 == 0, "a lane's loads must share the swizzle");
  int r0;   // this lane's row in load 0
  int col;  // element offset of the chunk it copies (source side)
  __device__ __forceinline__ void init(int w, int lane) {
    const int slot = w * 64 + lane;
    r0 = slot / CPR;
    col = ((slot % CPR) ^ (KV ? kv_swz<CPR>(r0) : bwd_swz<CPR>(r0))) * V;
  }
  __device__ __forceinline__ void issue(const T* __restrict__ g, int64_t S, int avail, T* lds, int w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int rr = min(r0 + i * STRIDE, avail - 1);
      __builtin_amdgcn_global_load_lds((bwd_glb_void*)(g + rr * S + col), (bwd_lds_void*)(lds + (4 * i + w) * 64 * V),
                                       16, 0, 0);
    }
  }
};

// 64 int64 timestamps ts[min(j, avail - 1)], j = 0..63, into LDS by one wave
// (two 4-byte-per-lane direct loads).
__device__ __forceinline__ void bwd_copy_ts(const int64_t* __restrict__ ts, int avail, int64_t* lds, int lane) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const int e = min(32 * d + (lane >> 1), avail - 1);
    __builtin_amdgcn_global_load_lds((bwd_glb_void*)(reinterpret_cast<const int32_t*>(ts + e) + (lane & 1)),
                                     (bwd_lds_void*)(lds + 32 * d), 4, 0, 0);
  }
}

// The earliest and latest timestamp of the 64-row block whose first row is
// `row` (the work list's per-block summary; a wave-uniform address, read-only
// here: scalar loads).
__device__ __forceinline__ void bwd_block_minmax(const int64_t* tstat, int64_t row, int64_t& mn, int64_t& mx) {
  const __attribute__((address_space(4))) int64_t* t4 =
      reinterpret_cast<const __attribute__((address_space(4))) int64_t*>(reinterpret_cast<uintptr_t>(tstat + 2 * row));
  mn = t4[0];
  mx = t4[1];
}

// Eight elements of one row in global memory, e0 .. e0 + 7.
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag bwd_global_frag(const T* p) {
  typedef typename Elem<T>::Frag Frag;
  if constexpr (Elem<T>::kVec == 8) {
    return *reinterpret_cast<const Frag*>(p);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    return Frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// A operand from tile rows: row r, elements e0 .. e0 + 7 (e0 a multiple of 8).
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::Frag bwd_row_frag(const T* lds, int r, int e0) {
  typedef typename Elem<T>::Frag Frag;
  typedef BTile<T, D> Bt;
  if constexpr (Elem<T>::kVec == 8) {
    return *reinterpret_cast<const Frag*>(lds + Bt::at(r, e0));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(lds + Bt::at(r, e0));
    const f32x4 b = *reinterpret_cast<const f32x4*>(lds + Bt::at(r, e0 + 4));
    return Frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

typedef short bwd_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bwd_v4i16 bwd_lds_v4i16;

// A operand from tile columns: feature f = 32 nt + lane % 32 of the eight rows
// kb + 8 (e / 4) + 4 half + e % 4 (the k order of an accumulator-fed B
// operand).  bf16: two transposing 8-byte LDS reads; within each 16-lane group
// of a ds_read_b64_tr_b16, lane l receives element l % 4 of the 4-element
// pieces addressed by lanes l / 4, 4 + l / 4, 8 + l / 4, 12 + l / 4, so lane a
// of the group addresses row kb + 4 half + a / 4, columns 32 nt + 16 ((lane /
// 16) % 2) + 4 (a % 4) .. + 3 (and the same 8 rows further).  fp32: element
// by element.
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::Frag bwd_col_frag(const T* lds, int kb, int nt, int lane) {
  typedef BTile<T, D> Bt;
  typename Elem<T>::Frag x;
  const int half = lane >> 5;
  if constexpr (Elem<T>::kVec == 8) {
    const int a = lane & 15;
    const int row = kb + 4 * half + (a >> 2);
    const int col = 32 * nt + 16 * ((lane >> 4) & 1) + 4 * (a & 3);
    const bwd_v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(lds + Bt::at(row, col)));
    const bwd_v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(lds + Bt::at(row + 8, col)));
    const bf16* p0 = reinterpret_cast<const bf16*>(&x0);
    const bf16* p1 = reinterpret_cast<const bf16*>(&x1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = p0[e];
      x[4 + e] = p1[e];
    }
  } else {
    const int f = 32 * nt + (lane & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = lds[Bt::at(kb + 8 * (e >> 2) + 4 * half + (e & 3), f)];
  }
  return x;
}

// Sixteen int64 timestamps from LDS: four groups of four consecutive
// entries, group q at p + q * STRIDE (p 16-byte aligned), read with eight
// 16-byte loads that are all issued before any result is used.
template <int STRIDE>
__device__ __forceinline__ void bwd_ts16(const int64_t* p, int64_t (&t)[16]) {
  typedef long long bwd_i64x2 __attribute__((ext_vector_type(2)));
  bwd_i64x2 v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const bwd_i64x2*>(p + (k >> 1) * STRIDE + 2 * (k & 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    t[2 * k] = v[k][0];
    t[2 * k + 1] = v[k][1];
  }
}

// Runs use(c, read(c)) for c = 0 .. N - 1 with the reads issued DEPTH
// steps ahead of their use, so that LDS latency overlaps the MFMAs.  The
// scheduling barriers keep the compiler from sinking each read back to its
// use, which it otherwise does to save registers.
template <int N, int DEPTH, typename Read, typename Use>
__device__ __forceinline__ void bwd_piped(Read read, Use use) {
  decltype(read(0)) buf[DEPTH];
#pragma unroll
  for (int c = 0; c < DEPTH && c < N; ++c) buf[c] = read(c);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const auto x = buf[c % DEPTH];
    use(c, x);
    if (c + DEPTH < N) buf[c % DEPTH] = read(c + DEPTH);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// An operand fragment of one tile row at precomputed element offsets: one
// 16-byte read for bf16, two for fp32 (offs[0], offs[1]).
template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag bwd_frag_at(const T* base, const int* offs) {
  typedef typename Elem<T>::Frag Frag;
  if constexpr (Elem<T>::kVec == 8) {
    return *reinterpret_cast<const Frag*>(base + offs[0]);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(base + offs[0]);
    const f32x4 b = *reinterpret_cast<const f32x4*>(base + offs[1]);
    return Frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// bwd_col_frag for bf16 at precomputed offsets of its two transposing reads.
__device__ __forceinline__ bf16x8 bwd_tr_frag(const bf16* base, const int* offs) {
  const bwd_v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(base + offs[0]));
  const bwd_v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(base + offs[1]));
  const bf16* p0 = reinterpret_cast<const bf16*>(&x0);
  const bf16* p1 = reinterpret_cast<const bf16*>(&x1);
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = p0[e];
    x[4 + e] = p1[e];
  }
  return x;
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag bwd_frag(const float* p) {
  typename Elem<T>::Frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = from_f32<T>(p[e]);
  return f;
}

__device__ __forceinline__ float bwd_sigmoid(float s) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(s * -1.4426950408889634f));
}

// Four gradient values of one token at flat index idx (row * N1 + column,
// column a multiple of 4) of the [T, N1] output: raw fp32 into dact, or (PRE)
// times SiLU'(pre) into dpre in the layer dtype.
template <typename T, bool PRE>
__device__ __forceinline__ void bwd_out4(const BwdArgs& a, int64_t idx, float x0, float x1, float x2, float x3) {
  if constexpr (PRE) {
    const T* p = reinterpret_cast<const T*>(a.pre) + idx;
    T* d = reinterpret_cast<T*>(a.dpre) + idx;
    if constexpr (sizeof(T) == 2) {
      const uint2 raw = *reinterpret_cast<const uint2*>(p);
      const T* z = reinterpret_cast<const T*>(&raw);
      T o[4] = {from_f32<T>(x0 * silu_grad(to_f32(z[0]))), from_f32<T>(x1 * silu_grad(to_f32(z[1]))),
                from_f32<T>(x2 * silu_grad(to_f32(z[2]))), from_f32<T>(x3 * silu_grad(to_f32(z[3])))};
      *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(o);
    } else {
      const float4 z = *reinterpret_cast<const float4*>(p);
      *reinterpret_cast<float4*>(d) =
          make_float4(x0 * silu_grad(z.x), x1 * silu_grad(z.y), x2 * silu_grad(z.z), x3 * silu_grad(z.w));
    }
  } else {
    *reinterpret_cast<float4*>(a.dact + idx) = make_float4(x0, x1, x2, x3);
  }
}

template <typename T, int DQK, int DV, bool PRE>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  typedef typename Elem<T>::Frag Frag;
  // two buffer sets (even / odd key blocks) of a K and a V tile, all in one
  // array so that each LDS read is a per-lane offset plus a constant
  constexpr int TK = 64 * DQK, SET = 64 * (DQK + DV);
  __shared__ __attribute__((aligned(16))) T tiles[2 * SET];
  __shared__ __attribute__((aligned(16))) int64_t tsks[2][64];
  // pos[P], time[NB], then one gradient histogram [P + NB] per wave (a
  // wave's updates land in program and lane order, so the sums are
  // reproducible; the four are added in wave order at the end)
  extern __shared__ float tabs[];
  const int H = a.H, h = blockIdx.x % H, item = blockIdx.x / H;
  const int P = a.P, NB = a.NB;
  float* pos_s = tabs;
  float* time_s = tabs + P;
  const int tid = threadIdx.x;
  if (item >= a.counts[0]) {  // whole workgroup: an empty partial row (rows past the items')
    float* part = a.tab_part + (int64_t)blockIdx.x * (P + NB);
    for (int i = tid; i < P + NB; i += 256) part[i] = 0.f;
    return;
  }
  // the tables times -log2(e): the weight step works on x = -log2(e) S
  for (int i = tid; i < P; i += 256)
    pos_s[i] = kNegLog2e * to_f32(reinterpret_cast<const T*>(a.pos_tab)[(int64_t)h * a.pos_stride + i]);
  for (int i = tid; i < NB; i += 256)
    time_s[i] = kNegLog2e * to_f32(reinterpret_cast<const T*>(a.time_tab)[(int64_t)h * a.time_stride + i]);
  for (int i = tid; i < 4 * (P + NB); i += 256) tabs[P + NB + i] = 0.f;
  float* gpos = tabs + (P + NB) * (1 + wave_id());
  float* gtime = gpos + P;
  const int2 tl = a.tiles[item];
  // The item's partial row is its stable index (sequence's first tile + its
  // query tile), so the column sums of table_grad_kernel add the same rows in
  // the same order whatever order the work list holds the items in.
  float* part = a.tab_part + ((int64_t)(a.tbase[tl.x] + tl.y) * H + h) * (P + NB);
  const SeqInfo si = seq_info(a.off, a.ncand, tl.x, a.T);
  const int L = si.len, nh = si.nhist;
  const int64_t s0 = si.start;
  const int i0 = tl.y * 128, iend = min(i0 + 128, L);
  const int lane = tid & 63, w = wave_id(), l32 = lane & 31, half = lane >> 5;
  const int r0 = i0 + 32 * w, iq = r0 + l32;
  const bool qvalid = iq < iend;
  // lanes without a row (they take no part in the wave's tests), and the
  // small-range bucket's bounds
  const uint64_t idle = ballot(!qvalid);
  const SmallBucket bk = small_bucket(a.NB, a.sbits);
  const float inv_n = 1.0f / (float)(a.norm_len > 0 ? a.norm_len : L);
  const int R = (P - 1) / 2;
  const bool shared = a.shared_pos != 0;
  const int K2 = H * DV;

  Frag qf[DQK / 16], df[DV / 16];
  const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)h * a.T + s0 + iq) * DQK;
  const T* drow = reinterpret_cast<const T*>(a.dout) + (s0 + iq) * (int64_t)K2 + h * DV;
#pragma unroll
  for (int c = 0; c < DQK / 16; ++c) {
    qf[c] = Frag{};
    if (qvalid) qf[c] = bwd_global_frag<T>(qrow + 16 * c + 8 * half);
  }
#pragma unroll
  for (int c = 0; c < DV / 16; ++c) {
    df[c] = Frag{};
    if (qvalid) df[c] = bwd_global_frag<T>(drow + 16 * c + 8 * half);
  }
  const int p_q = position(iq, nh, shared);
  const int64_t ts_q = qvalid ? a.ts[s0 + iq] : 0;
  // Bias-gradient aggregation per lane before the LDS histograms: the two
  // clamped position buckets (0 and 2R, every pair at distance >= R) add up
  // in registers, and each time bucket in a run of equal buckets (a lane's
  // keys advance in time, so its buckets change rarely) is added once.
  float far_lo = 0.f, far_hi = 0.f, run = 0.f;
  int run_bt = 0;
  f32x16 dq[DQK / 32];
#pragma unroll
  for (int n = 0; n < DQK / 32; ++n) dq[n] = f32x16{};

  // key blocks: the history up to the tile's last row, then the blocks with
  // the tile's candidates' own keys
  const int a_end = min(iend, nh);
  const int nblk_a = (a_end + 63) / 64;
  const int b_lo = max(i0, nh);
  const int jb0 = max(nblk_a * 64, (b_lo / 64) * 64);
  const int nblk_b = (b_lo < iend && jb0 < iend) ? (iend - jb0 + 63) / 64 : 0;
  const T* kg = reinterpret_cast<const T*>(a.k) + ((int64_t)h * a.T + s0) * DQK;
  const T* vg = reinterpret_cast<const T*>(a.v) + ((int64_t)h * a.T + s0) * DV;
  const int nblk = nblk_a + nblk_b;
  auto block_start = [&](int blk) __attribute__((always_inline)) {
    return blk < nblk_a ? blk * 64 : jb0 + (blk - nblk_a) * 64;
  };
  BwdCopy<T, DQK> kcopy;
  BwdCopy<T, DV> vcopy;
  kcopy.init(w, lane);
  vcopy.init(w, lane);
  // Per-lane LDS offsets of the fragment reads for the tile's rows 0..31
  // (row l32) and, for bf16, of dQ's transposing reads at key rows 0..15:
  // rows further by a multiple of 16 add a constant, the swizzle depending on
  // the row modulo 16 only.
  constexpr int RW = Elem<T>::kVec == 8 ? 1 : 2;
  int rk[DQK / 16][RW], rv[DV / 16][RW], ck[DQK / 32][2];
#pragma unroll
  for (int c = 0; c < DQK / 16; ++c)
#pragma unroll
    for (int u = 0; u < RW; ++u) rk[c][u] = BTile<T, DQK>::at(l32, 16 * c + 8 * half + 4 * u);
#pragma unroll
  for (int c = 0; c < DV / 16; ++c)
#pragma unroll
    for (int u = 0; u < RW; ++u) rv[c][u] = BTile<T, DV>::at(l32, 16 * c + 8 * half + 4 * u);
#pragma unroll
  for (int n = 0; n < DQK / 32; ++n) {
    const int a4 = lane & 15, row = 4 * half + (a4 >> 2), col = 32 * n + 16 * ((lane >> 4) & 1) + 4 * (a4 & 3);
    ck[n][0] = BTile<T, DQK>::at(row, col);
    ck[n][1] = BTile<T, DQK>::at(row + 8, col);
  }
  // K, V rows and key timestamps of block blk into one buffer set
  auto issue = [&](int blk, int set) __attribute__((always_inline)) {
    T* Ks = tiles + set * SET;
    T* Vs = Ks + TK;
    int64_t* tsk = tsks[set];
    const int j0 = block_start(blk);
    kcopy.issue(kg + (int64_t)j0 * DQK, DQK, L - j0, Ks, w);
    vcopy.issue(vg + (int64_t)j0 * DV, DV, L - j0, Vs, w);
    if (w == 0) bwd_copy_ts(a.ts + s0 + j0, L - j0, tsk, lane);
  };
  auto consume = [&](int blk, int set) __attribute__((always_inline)) {
    const T* Ks = tiles + set * SET;
    const T* Vs = Ks + TK;
    const int64_t* tsk = tsks[set];
    const int j0 = block_start(blk);
    if (r0 >= iend) return;
    // A far block: every key a history key strictly before the wave's first
    // row and at least R positions from it (position bucket 2R, no mask).
    // Per row the block's time differences lie in [ts_q - kmax, ts_q - kmin]
    // (no overflow) and the bucket is monotone in dt: with one bucket at both
    // ends the bias is one value per row (mode 0); with two adjacent ones a
    // key takes the upper bucket exactly when ts_j <= ts_q - (first dt of
    // that bucket) (mode 1).  Otherwise every pair is bucketed (mode 2).
    // The mode is wave-uniform.
    // Mode 2 takes each pair's time difference from the low 32 bits of both
    // timestamps when every row's range lies within +-2^24 (small).
    const bool far = j0 + 63 < L && j0 + 63 < nh && j0 + 63 < r0 && position(r0, nh, shared) - (j0 + 63) >= R;
    int mode = 2, bt_lo = 0, bt_hi = 0;
    float b_lo = 0.f, b_hi = 0.f;
    int64_t tcut = 0, kmin, kmax, dlo, dhi;
    bwd_block_minmax(a.tstat, s0 + j0, kmin, kmax);
    const bool ok = !__builtin_sub_overflow(ts_q, kmax, &dlo) && !__builtin_sub_overflow(ts_q, kmin, &dhi);
    const uint64_t okm = ballot(ok);
    const bool small = all_lanes((okm & ballot(dlo > -(1 << 24)) & ballot(dhi < (1 << 24))) | idle);
    if (far) {
      bt_lo = small ? time_bucket_med3((int)dlo, bk) : time_bucket(dlo, NB, a.sbits);
      bt_hi = small ? time_bucket_med3((int)dhi, bk) : time_bucket(dhi, NB, a.sbits);
      b_lo = pos_s[2 * R] + time_s[bt_lo];
      if (all_lanes((okm & ballot(bt_lo == bt_hi)) | idle)) {
        mode = 0;
      } else if (all_lanes((okm & ballot(bt_hi <= bt_lo + 1)) | idle)) {
        mode = 1;
        b_hi = pos_s[2 * R] + time_s[bt_hi];
        tcut = ts_q - bucket_floor(max(bt_hi, 1), a.sbits);  // >= kmin: no overflow
      }
      mode = __builtin_amdgcn_readfirstlane(mode);
    }
    // dS_ij N_b = dA_ij SiLU'(S_ij) from x = -log2(e) S_ij: sg = 1 / (1 + 2^x),
    // SiLU'(S) = sg + S sg (1 - sg) = (x sg) ln2 (sg - 1) + sg; a masked pair
    // gets x = 1e30 (sg = 0, dS = 0).  1 / N_b is applied to dQ and to the
    // table-gradient row at the end.  The dQ columns of rows past the tile
    // are never stored, so only their table-gradient sums are masked.
    auto dsv = [](float d, float x) __attribute__((always_inline)) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
      return d * __builtin_fmaf(x * sg, __builtin_fmaf(sg, -kNegLn2, kNegLn2), sg);
    };
    // time-bucket gradient runs: a lane's buckets only fall as its keys advance
    auto add_run = [&](int bt, float v) __attribute__((always_inline)) {
      if (bt != run_bt) {
        if (run != 0.f) atomicAdd(&gtime[run_bt], run);
        run_bt = bt;
        run = 0.f;
      }
      run += v;
    };
    // Mode 2: each pair's buckets, mask and table-gradient updates
    auto pairs = [&](auto small_t, int kh, const f32x16& sc, const f32x16& da, float (&ds)[16])
                     __attribute__((always_inline)) {
      constexpr bool SMALL = decltype(small_t)::value;
      int64_t tk[16];
      bwd_ts16<8>(tsk + kh * 32 + 4 * half, tk);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3), j = j0 + kl;
        const bool valid = qvalid && j < L && attends(iq, j, nh);
        const int bp = pos_bucket(p_q, position(j, nh, shared), R);
        const int bt = SMALL ? time_bucket_med3((int)((uint32_t)ts_q - (uint32_t)tk[r]), bk)
                             : time_bucket(wrap_sub(ts_q, tk[r]), NB, a.sbits);
        const float g = dsv(da[r], valid ? __builtin_fmaf(sc[r], kNegLog2e, pos_s[bp] + time_s[bt]) : 1e30f);
        ds[r] = g;
        if (valid) {
          if (bp == 0)
            far_lo += g;
          else if (bp == 2 * R)
            far_hi += g;
          else
            atomicAdd(&gpos[bp], g);
          add_run(bt, g);
        }
      }
    };
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x16 sc = f32x16{}, da = f32x16{};
      // S^T then dA^T: K rows, then V rows, read four steps ahead
      constexpr int NK = DQK / 16, NV = DV / 16;
      bwd_piped<NK + NV, 4>(
          [&](int c) __attribute__((always_inline)) {
            return c < NK ? bwd_frag_at<T>(Ks + kh * 32 * DQK, rk[c]) : bwd_frag_at<T>(Vs + kh * 32 * DV, rv[c - NK]);
          },
          [&](int c, const Frag& x) __attribute__((always_inline)) {
            if (c < NK)
              sc = mma_k16(x, qf[c], sc);
            else
              da = mma_k16(x, df[c - NK], da);
          });
      float ds[16];
      if (mode == 0) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          ds[r] = dsv(da[r], __builtin_fmaf(sc[r], kNegLog2e, b_lo));
          sum += ds[r];
        }
        sum = qvalid ? sum : 0.f;
        far_hi += sum;
        add_run(bt_lo, sum);
      } else if (mode == 1) {
        float sum_lo = 0.f, sum_hi = 0.f;
        int64_t tk[16];  // element r: key kh * 32 + 8 (r / 4) + 4 half + r % 4
        bwd_ts16<8>(tsk + kh * 32 + 4 * half, tk);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool up = tk[r] <= tcut;
          ds[r] = dsv(da[r], __builtin_fmaf(sc[r], kNegLog2e, up ? b_hi : b_lo));
          sum_hi += up ? ds[r] : 0.f;
          sum_lo += up ? 0.f : ds[r];
        }
        sum_hi = qvalid ? sum_hi : 0.f;
        sum_lo = qvalid ? sum_lo : 0.f;
        far_hi += sum_hi + sum_lo;
        add_run(bt_hi, sum_hi);
        add_run(bt_lo, sum_lo);
      } else if (small) {
        pairs(std::true_type{}, kh, sc, da, ds);
      } else {
        pairs(std::false_type{}, kh, sc, da, ds);
      }
      // dQ^T += K^T dS^T over the two 16-key halves, K^T read two steps ahead
      constexpr int NQ = DQK / 32;
      const Frag pf0 = bwd_frag<T>(ds), pf1 = bwd_frag<T>(ds + 8);
      bwd_piped<2 * NQ, 2>(
          [&](int c) __attribute__((always_inline)) {
            const int c2 = c / NQ, n = c % NQ;
            if constexpr (Elem<T>::kVec == 8)
              return bwd_tr_frag(Ks + (kh * 32 + 16 * c2) * DQK, ck[n]);
            else
              return bwd_col_frag<T, DQK>(Ks, kh * 32 + 16 * c2, n, lane);
          },
          [&](int c, const Frag& x) __attribute__((always_inline)) {
            dq[c % NQ] = mma_k16(x, c < NQ ? pf0 : pf1, dq[c % NQ]);
          });
    }
  };
  if (nblk > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block 0 have landed
  __syncthreads();                // ... and every wave's, plus the tables and histograms
  // Two blocks per trip so that each buffer set is named by a constant: the
  // copies of block b + 1 run while block b is consumed; one barrier per block.
  for (int blk = 0; blk < nblk; blk += 2) {
    if (blk + 1 < nblk) issue(blk + 1, 1);
    consume(blk, 0);
    if (blk + 1 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (blk + 2 < nblk) issue(blk + 2, 0);
    consume(blk + 1, 1);
    if (blk + 2 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (qvalid) {
    const int64_t dst = (s0 + iq) * (int64_t)a.N1 + 2 * K2 + h * DQK + 4 * half;
#pragma unroll
    for (int n = 0; n < DQK / 32; ++n)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        bwd_out4<T, PRE>(a, dst + 32 * n + 8 * g4, inv_n * dq[n][4 * g4], inv_n * dq[n][4 * g4 + 1],
                         inv_n * dq[n][4 * g4 + 2], inv_n * dq[n][4 * g4 + 3]);
  }
  if (run != 0.f) atomicAdd(&gtime[run_bt], run);
  if (far_lo != 0.f) atomicAdd(&gpos[0], far_lo);
  if (far_hi != 0.f) atomicAdd(&gpos[2 * R], far_hi);
  __syncthreads();  // every LDS histogram update is done
  for (int i = tid; i < P + NB; i += 256) {
    const float* hw = tabs + (P + NB) + i;
    part[i] = inv_n * (((hw[0] + hw[P + NB]) + hw[2 * (P + NB)]) + hw[3 * (P + NB)]);
  }
}

template <typename T, int DQK, int DV, bool DK, bool PRE>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_kernel(BwdArgs a) {
  typedef typename Elem<T>::Frag Frag;
  constexpr int DACC = DK ? DQK : DV;  // width of this pass's gradient
  // two buffer sets (even / odd query blocks), each its own LDS objects
  __shared__ __attribute__((aligned(16))) T Qs0[64 * DQK];
  __shared__ __attribute__((aligned(16))) T Qs1[64 * DQK];
  __shared__ __attribute__((aligned(16))) T Os0[64 * DV];
  __shared__ __attribute__((aligned(16))) T Os1[64 * DV];
  __shared__ __attribute__((aligned(16))) int64_t tsq0[64];
  __shared__ __attribute__((aligned(16))) int64_t tsq1[64];
  extern __shared__ float tabs[];  // pos[P], time[NB]
  const int H = a.H, h = blockIdx.x % H, item = blockIdx.x / H;
  if (item >= a.counts[0]) return;
  const int P = a.P, NB = a.NB;
  float* pos_s = tabs;
  float* time_s = tabs + P;
  const int tid = threadIdx.x;
  for (int i = tid; i < P; i += 256)
    pos_s[i] = to_f32(reinterpret_cast<const T*>(a.pos_tab)[(int64_t)h * a.pos_stride + i]);
  for (int i = tid; i < NB; i += 256)
    time_s[i] = to_f32(reinterpret_cast<const T*>(a.time_tab)[(int64_t)h * a.time_stride + i]);
  const int2 tl = a.tiles[item];
  const SeqInfo si = seq_info(a.off, a.ncand, tl.x, a.T);
  const int L = si.len, nh = si.nhist;
  const int64_t s0 = si.start;
  const int j0t = tl.y * 128, jend = min(j0t + 128, L);
  const int lane = tid & 63, w = wave_id(), l32 = lane & 31, half = lane >> 5;
  const int kr0 = j0t + 32 * w, jk = kr0 + l32;
  const bool kvalid = jk < jend;
  // lanes without a row (they take no part in the wave's tests), and the
  // small-range bucket's bounds
  const uint64_t idle = ballot(!kvalid);
  const SmallBucket bk = small_bucket(a.NB, a.sbits);
  const float inv_n = 1.0f / (float)(a.norm_len > 0 ? a.norm_len : L);
  const int R = (P - 1) / 2;
  const bool shared = a.shared_pos != 0;
  const int K2 = H * DV;

  Frag kf[DQK / 16], vf[DK ? DV / 16 : 1];
  const T* krow = reinterpret_cast<const T*>(a.k) + ((int64_t)h * a.T + s0 + jk) * DQK;
  const T* vrow = reinterpret_cast<const T*>(a.v) + ((int64_t)h * a.T + s0 + jk) * DV;
#pragma unroll
  for (int c = 0; c < DQK / 16; ++c) {
    kf[c] = Frag{};
    if (kvalid) kf[c] = bwd_global_frag<T>(krow + 16 * c + 8 * half);
  }
  if (DK) {
#pragma unroll
    for (int c = 0; c < DV / 16; ++c) {
      vf[c] = Frag{};
      if (kvalid) vf[c] = bwd_global_frag<T>(vrow + 16 * c + 8 * half);
    }
  }
  const int p_k = position(jk, nh, shared);
  const int64_t ts_k = kvalid ? a.ts[s0 + jk] : 0;
  f32x16 acc[DACC / 32];
#pragma unroll
  for (int n = 0; n < DACC / 32; ++n) acc[n] = f32x16{};

  // query blocks: history keys are seen by every later row (candidates
  // included); candidate keys only by their own row
  const int qb0 = (j0t / 64) * 64;
  const int qend = j0t < nh ? L : jend;
  const T* qg = reinterpret_cast<const T*>(a.q) + ((int64_t)h * a.T + s0) * DQK;
  const T* og = reinterpret_cast<const T*>(a.dout) + s0 * (int64_t)K2 + h * DV;
  const int nblk = qend > qb0 ? (qend - qb0 + 63) / 64 : 0;
  BwdCopy<T, DQK> qcopy;
  BwdCopy<T, DV> ocopy;
  qcopy.init(w, lane);
  ocopy.init(w, lane);
  // Q, dO rows and query timestamps of query block blk into one buffer set
  auto issue = [&](int blk, T* Qs, T* Os, int64_t* tsq) __attribute__((always_inline)) {
    const int i0 = qb0 + 64 * blk;
    qcopy.issue(qg + (int64_t)i0 * DQK, DQK, L - i0, Qs, w);
    ocopy.issue(og + (int64_t)i0 * K2, K2, L - i0, Os, w);
    if (w == 0) bwd_copy_ts(a.ts + s0 + i0, L - i0, tsq, lane);
  };
  auto consume = [&](int blk, const T* Qs, const T* Os, const int64_t* tsq) __attribute__((always_inline)) {
    const int i0 = qb0 + 64 * blk;
    if (kr0 >= jend) return;
    // A far block (the dq kernel's test with queries and keys swapped): all
    // the wave's keys history keys strictly before the block's first query
    // and at least R positions from it; one time bucket per key.
    // Modes as in the dq kernel, per key: the block's differences lie in
    // [qmin - ts_k, qmax - ts_k]; in mode 1 a query takes the upper bucket
    // exactly when ts_i >= ts_k + (first dt of that bucket).
    const int k_last = min(kr0 + 31, jend - 1);
    const bool far = i0 + 63 < L && k_last < nh && i0 > k_last && position(i0, nh, shared) - k_last >= R;
    int mode = 2;
    float b_lo = 0.f, b_hi = 0.f;
    int64_t tcut = 0, qmin, qmax, dlo, dhi;
    bwd_block_minmax(a.tstat, s0 + i0, qmin, qmax);
    const bool ok = !__builtin_sub_overflow(qmin, ts_k, &dlo) && !__builtin_sub_overflow(qmax, ts_k, &dhi);
    const uint64_t okm = ballot(ok);
    const bool small = all_lanes((okm & ballot(dlo > -(1 << 24)) & ballot(dhi < (1 << 24))) | idle);
    // Mode 2: each pair's buckets and mask (32-bit differences when small)
    auto pairs = [&](auto small_t, int qh, const f32x16& sc, const f32x16& da, float (&g)[16])
                     __attribute__((always_inline)) {
      constexpr bool SMALL = decltype(small_t)::value;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qh * 32 + 8 * (r >> 2) + 4 * half + (r & 3), i = i0 + ql;
        const bool valid = kvalid && i < L && attends(i, jk, nh);
        const int bp = pos_bucket(position(i, nh, shared), p_k, R);
        const int bt = SMALL ? time_bucket_med3((int)((uint32_t)tsq[ql] - (uint32_t)ts_k), bk)
                             : time_bucket(wrap_sub(tsq[ql], ts_k), NB, a.sbits);
        const float s = sc[r] + pos_s[bp] + time_s[bt];
        const float sg = bwd_sigmoid(s);
        const float val = DK ? da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n : s * sg * inv_n;
        g[r] = valid ? val : 0.f;
      }
    };
    if (far) {
      const int lo = small ? time_bucket_med3((int)dlo, bk) : time_bucket(dlo, NB, a.sbits);
      const int hi = small ? time_bucket_med3((int)dhi, bk) : time_bucket(dhi, NB, a.sbits);
      b_lo = pos_s[2 * R] + time_s[lo];
      if (all_lanes((okm & ballot(lo == hi)) | idle)) {
        mode = 0;
      } else if (all_lanes((okm & ballot(hi <= lo + 1)) | idle)) {
        mode = 1;
        b_hi = pos_s[2 * R] + time_s[hi];
        tcut = ts_k + bucket_floor(max(hi, 1), a.sbits);  // <= qmax: no overflow
      }
      mode = __builtin_amdgcn_readfirstlane(mode);
    }
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      f32x16 sc = f32x16{}, da = f32x16{};
#pragma unroll
      for (int c = 0; c < DQK / 16; ++c) sc = mma_k16(bwd_row_frag<T, DQK>(Qs, qh * 32 + l32, 16 * c + 8 * half), kf[c], sc);
      if (DK) {
#pragma unroll
        for (int c = 0; c < DV / 16; ++c) da = mma_k16(bwd_row_frag<T, DV>(Os, qh * 32 + l32, 16 * c + 8 * half), vf[c], da);
      }
      float g[16];
      if (mode == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sc[r] + b_lo;
          const float sg = bwd_sigmoid(s);
          const float val = DK ? da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n : s * sg * inv_n;
          g[r] = kvalid ? val : 0.f;
        }
      } else if (mode == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qh * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float s = sc[r] + (tsq[ql] >= tcut ? b_hi : b_lo);
          const float sg = bwd_sigmoid(s);
          const float val = DK ? da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n : s * sg * inv_n;
          g[r] = kvalid ? val : 0.f;
        }
      } else if (small) {
        pairs(std::true_type{}, qh, sc, da, g);
      } else {
        pairs(std::false_type{}, qh, sc, da, g);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const Frag pf = bwd_frag<T>(g + 8 * c2);
#pragma unroll
        for (int n = 0; n < DACC / 32; ++n) {
          const Frag af = DK ? bwd_col_frag<T, DQK>(Qs, qh * 32 + 16 * c2, n, lane)
                             : bwd_col_frag<T, DV>(Os, qh * 32 + 16 * c2, n, lane);
          acc[n] = mma_k16(af, pf, acc[n]);
        }
      }
    }
  };
  if (nblk > 0) issue(0, Qs0, Os0, tsq0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block 0 have landed
  __syncthreads();                // ... and every wave's, plus the tables
  // Two blocks per trip so that each buffer set is named by a constant: the
  // copies of block b + 1 run while block b is consumed; one barrier per block.
  for (int blk = 0; blk < nblk; blk += 2) {
    if (blk + 1 < nblk) issue(blk + 1, Qs1, Os1, tsq1);
    consume(blk, Qs0, Os0, tsq0);
    if (blk + 1 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (blk + 2 < nblk) issue(blk + 2, Qs0, Os0, tsq0);
    consume(blk + 1, Qs1, Os1, tsq1);
    if (blk + 2 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (kvalid) {
    const int64_t dst =
        (s0 + jk) * (int64_t)a.N1 + (DK ? 2 * K2 + H * DQK + h * DQK : K2 + h * DV) + 4 * half;
#pragma unroll
    for (int n = 0; n < DACC / 32; ++n)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        bwd_out4<T, PRE>(a, dst + 32 * n + 8 * g4, acc[n][4 * g4], acc[n][4 * g4 + 1], acc[n][4 * g4 + 2],
                         acc[n][4 * g4 + 3]);
  }
}

// One 16 x 16 x 32 bf16 MFMA step.  Lane l holds A row l % 16 and B column
// l % 16 at k values 8 (l / 16) .. + 7, and C column l % 16 at rows
// 4 (l / 16) .. + 3.
__device__ __forceinline__ f32x4 mma16(const bf16x8& x, const bf16x8& y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
}

// A operand of a 16 x 16 x 32 step from tile columns: A row m = feature
// 16 ft + m (m = lane % 16); k value e = tile row kb + 4 (lane / 16) + e for
// e < 4 and kb + 16 + 4 (lane / 16) + e - 4 above, the order in which a lane
// holds the accumulator rows of two consecutive 16-row tiles.  Two
// transposing 8-byte reads: within each 16-lane group, lane a addresses row
// kb + 4 (lane / 16) + a / 4, columns 16 ft + 4 (a % 4) .. + 3, and receives
// column 16 ft + a of the group's four rows (then the same 16 rows further).
// kv_col_off is the lane's element offset for kb = 0; kb, a multiple of 16,
// adds kb D (the swizzle depends on the row modulo 16), so one offset register
// per ft serves every row block and, with the tiles in one array, every tile.
template <int D>
__device__ __forceinline__ int kv_col_off(int lane, int ft) {
  const int a = lane & 15;
  return KvTile<D>::at(4 * (lane >> 4) + (a >> 2), 16 * ft + 4 * (a & 3));
}
template <int D>
__device__ __forceinline__ bf16x8 kv_col_frag(const bf16* p) {
  const bwd_v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)p);
  const bwd_v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(p + 16 * D));
  const bf16* p0 = reinterpret_cast<const bf16*>(&x0);
  const bf16* p1 = reinterpret_cast<const bf16*>(&x1);
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = p0[e];
    x[4 + e] = p1[e];
  }
  return x;
}

// attn_bwd_kv16_kernel (bf16): dK and dV in one pass.  Work item (sequence,
// 64-key half of a 128-key tile, head); each of the four waves owns 16 keys
// and keeps both gradients in registers on 16 x 16 x 32 MFMA tiles (half the
// accumulator registers per key of 32 x 32 tiles), so S = Q K^T, dA = dO V^T
// and the weights are formed once per (key, query block) rather than once per
// gradient.  Per query block of 64 rows: four 16-query tiles of S and dA (Q,
// dO rows from LDS, K, V in registers), then dV^T += dO^T a and
// dK^T += Q^T dS with a and dS fed from the accumulators as the B operand.
template <int DQK, int DV, bool PRE>
__global__ __launch_bounds__(256, 2) void attn_bwd_kv16_kernel(BwdArgs a) {
  typedef bf16 T;
  // two buffer sets (even / odd query blocks) of a Q and a dO tile, all in
  // one array so that each LDS read is a per-lane offset plus a constant
  constexpr int TQ = 64 * DQK, SET = 64 * (DQK + DV);
  __shared__ __attribute__((aligned(16))) T tiles[2 * SET];
  __shared__ __attribute__((aligned(16))) int64_t tsqs[2][64];
  extern __shared__ float tabs[];  // pos[P], time[NB]
  const int H = a.H, h = blockIdx.x % H, unit = blockIdx.x / H, item = unit >> 1;
  if (item >= a.counts[0]) return;
  const int2 tl = a.tiles[item];
  const SeqInfo si = seq_info(a.off, a.ncand, tl.x, a.T);
  const int L = si.len, nh = si.nhist;
  const int j0t = tl.y * 128 + 64 * (unit & 1);
  if (j0t >= L) return;  // the tile's second half lies past the sequence
  const int P = a.P, NB = a.NB;
  float* pos_s = tabs;
  float* time_s = tabs + P;
  const int tid = threadIdx.x;
  // the tables times -log2(e): the weight step works on x = -log2(e) S
  for (int i = tid; i < P; i += 256)
    pos_s[i] = kNegLog2e * to_f32(reinterpret_cast<const T*>(a.pos_tab)[(int64_t)h * a.pos_stride + i]);
  for (int i = tid; i < NB; i += 256)
    time_s[i] = kNegLog2e * to_f32(reinterpret_cast<const T*>(a.time_tab)[(int64_t)h * a.time_stride + i]);
  const int64_t s0 = si.start;
  const int jend = min(j0t + 64, L);
  const int lane = tid & 63, w = wave_id(), g = lane >> 4, l16 = lane & 15;
  const int kr0 = j0t + 16 * w, jk = kr0 + l16;
  const bool kvalid = jk < jend;
  // lanes without a row (they take no part in the wave's tests), and the
  // small-range bucket's bounds
  const uint64_t idle = ballot(!kvalid);
  const SmallBucket bk = small_bucket(a.NB, a.sbits);
  const float inv_n = 1.0f / (float)(a.norm_len > 0 ? a.norm_len : L);
  const int R = (P - 1) / 2;
  const bool shared = a.shared_pos != 0;
  const int K2 = H * DV;

  // S and dA contract over the head dimension in the chunk order kv_chunk:
  // k-step c takes 16-byte chunk c + (D / 32) g for lane group g, which keeps
  // the 16-row reads of Q and dO free of bank conflicts (adjacent chunks per
  // group conflict two-way under kv_swz, measured); K and V use the same order
  bf16x8 kf[DQK / 32], vf[DV / 32];
  const T* krow = reinterpret_cast<const T*>(a.k) + ((int64_t)h * a.T + s0 + jk) * DQK;
  const T* vrow = reinterpret_cast<const T*>(a.v) + ((int64_t)h * a.T + s0 + jk) * DV;
#pragma unroll
  for (int c = 0; c < DQK / 32; ++c) {
    kf[c] = bf16x8{};
    if (kvalid) kf[c] = bwd_global_frag<T>(krow + 8 * (c + (DQK / 32) * g));
  }
#pragma unroll
  for (int c = 0; c < DV / 32; ++c) {
    vf[c] = bf16x8{};
    if (kvalid) vf[c] = bwd_global_frag<T>(vrow + 8 * (c + (DV / 32) * g));
  }
  const int p_k = position(jk, nh, shared);
  const int64_t ts_k = kvalid ? a.ts[s0 + jk] : 0;
  f32x4 dk[DQK / 16], dv[DV / 16];
#pragma unroll
  for (int n = 0; n < DQK / 16; ++n) dk[n] = f32x4{};
#pragma unroll
  for (int n = 0; n < DV / 16; ++n) dv[n] = f32x4{};

  // query blocks: history keys are seen by every later row (candidates
  // included); candidate keys only by their own row
  const int qend = j0t < nh ? L : jend;
  const T* qg = reinterpret_cast<const T*>(a.q) + ((int64_t)h * a.T + s0) * DQK;
  const T* og = reinterpret_cast<const T*>(a.dout) + s0 * (int64_t)K2 + h * DV;
  const int nblk = (qend - j0t + 63) / 64;
  BwdCopy<T, DQK, true> qcopy;
  BwdCopy<T, DV, true> ocopy;
  qcopy.init(w, lane);
  ocopy.init(w, lane);
  int roq[DQK / 32], rov[DV / 32], coq[DQK / 16], cov[DV / 16];  // per-lane LDS offsets
#pragma unroll
  for (int c = 0; c < DQK / 32; ++c) roq[c] = KvTile<DQK>::at(l16, 8 * (c + (DQK / 32) * g));
#pragma unroll
  for (int c = 0; c < DV / 32; ++c) rov[c] = KvTile<DV>::at(l16, 8 * (c + (DV / 32) * g));
#pragma unroll
  for (int ft = 0; ft < DQK / 16; ++ft) coq[ft] = kv_col_off<DQK>(lane, ft);
#pragma unroll
  for (int ft = 0; ft < DV / 16; ++ft) cov[ft] = kv_col_off<DV>(lane, ft);
  auto issue = [&](int blk, int set) __attribute__((always_inline)) {
    T* Qs = tiles + set * SET;
    T* Os = Qs + TQ;
    int64_t* tsq = tsqs[set];
    const int i0 = j0t + 64 * blk;
    qcopy.issue(qg + (int64_t)i0 * DQK, DQK, L - i0, Qs, w);
    ocopy.issue(og + (int64_t)i0 * K2, K2, L - i0, Os, w);
    if (w == 0) bwd_copy_ts(a.ts + s0 + i0, L - i0, tsq, lane);
  };
  auto consume = [&](int blk, int set) __attribute__((always_inline)) {
    const T* Qs = tiles + set * SET;
    const T* Os = Qs + TQ;
    const int64_t* tsq = tsqs[set];
    const int i0 = j0t + 64 * blk;
    if (kr0 >= jend) return;
    // Weight modes per (wave, query block) as in attn_bwd_dkv_kernel, over
    // the wave's 16 keys.
    const int k_last = min(kr0 + 15, jend - 1);
    const bool far = i0 + 63 < L && k_last < nh && i0 > k_last && position(i0, nh, shared) - k_last >= R;
    int mode = 2;
    float b_lo = 0.f, b_hi = 0.f;
    int64_t tcut = 0, qmin, qmax, dlo, dhi;
    bwd_block_minmax(a.tstat, s0 + i0, qmin, qmax);
    const bool ok = !__builtin_sub_overflow(qmin, ts_k, &dlo) && !__builtin_sub_overflow(qmax, ts_k, &dhi);
    const uint64_t okm = ballot(ok);
    const bool small = all_lanes((okm & ballot(dlo > -(1 << 24)) & ballot(dhi < (1 << 24))) | idle);
    if (far) {
      const int lo = small ? time_bucket_med3((int)dlo, bk) : time_bucket(dlo, NB, a.sbits);
      const int hi = small ? time_bucket_med3((int)dhi, bk) : time_bucket(dhi, NB, a.sbits);
      b_lo = pos_s[2 * R] + time_s[lo];
      if (all_lanes((okm & ballot(lo == hi)) | idle)) {
        mode = 0;
      } else if (all_lanes((okm & ballot(hi <= lo + 1)) | idle)) {
        mode = 1;
        b_hi = pos_s[2 * R] + time_s[hi];
        tcut = ts_k + bucket_floor(max(hi, 1), a.sbits);  // <= qmax: no overflow
      }
      mode = __builtin_amdgcn_readfirstlane(mode);
    }
    // S and dA over the block's four 16-query tiles; element e = 4 qt + r of
    // a lane is query i0 + 16 qt + 4 g + r, key jk
    f32x4 sc[4], da[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) sc[qt] = da[qt] = f32x4{};
    // step t: S (t < 4 NK) or dA, query tile t % 4, k chunk (t / 4) % NK;
    // consecutive steps use different accumulators
    constexpr int NK = DQK / 32, NV = DV / 32;
    bwd_piped<4 * (NK + NV), 4>(
        [&](int t) __attribute__((always_inline)) {
          const int qt = t % 4, c = (t / 4) % (t < 4 * NK ? NK : NV);
          return t < 4 * NK ? *reinterpret_cast<const bf16x8*>(Qs + 16 * qt * DQK + roq[c])
                            : *reinterpret_cast<const bf16x8*>(Os + 16 * qt * DV + rov[c]);
        },
        [&](int t, const bf16x8& x) __attribute__((always_inline)) {
          const int qt = t % 4;
          if (t < 4 * NK)
            sc[qt] = mma16(x, kf[(t / 4) % NK], sc[qt]);
          else
            da[qt] = mma16(x, vf[(t / 4 - NK) % NV], da[qt]);
        });
    // Weight step on x = -log2(e) S_ij (a masked pair gets x = 1e30):
    //   sg = sigmoid(S) = 1 / (1 + 2^x),  t = x sg = -log2(e) SiLU(S),
    //   SiLU'(S) = sg + SiLU(S) (1 - sg) = t u + sg with u = ln2 (sg - 1).
    // The B operands hold t and dA SiLU'(S); the constant factors -ln2 / N_b
    // and 1 / N_b are applied to the accumulators once, at the end.  A masked
    // pair gives 2^x = inf, sg = 0, t = 0 and SiLU' = 0.  Keys past the tile
    // need no mask: their K and V rows are zero and their accumulator columns
    // are never stored.
    float pa[16], pd[16];
    auto put = [&](int e, float x) __attribute__((always_inline)) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
      const float t = x * sg;
      pa[e] = t;
      pd[e] = da[e >> 2][e & 3] * __builtin_fmaf(t, __builtin_fmaf(sg, -kNegLn2, kNegLn2), sg);
    };
    // mode 2: each pair's buckets and mask (32-bit differences when small)
    auto pairs = [&](auto small_t) __attribute__((always_inline)) {
      constexpr bool SMALL = decltype(small_t)::value;
      int64_t tq[16];
      bwd_ts16<16>(tsq + 4 * g, tq);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ql = 16 * (e >> 2) + 4 * g + (e & 3), i = i0 + ql;
        const bool valid = kvalid && i < L && attends(i, jk, nh);
        const int bp = pos_bucket(position(i, nh, shared), p_k, R);
        const int bt = SMALL ? time_bucket_med3((int)((uint32_t)tq[e] - (uint32_t)ts_k), bk)
                             : time_bucket(wrap_sub(tq[e], ts_k), NB, a.sbits);
        const float x = __builtin_fmaf(sc[e >> 2][e & 3], kNegLog2e, pos_s[bp] + time_s[bt]);
        put(e, valid ? x : 1e30f);
      }
    };
    if (mode == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) put(e, __builtin_fmaf(sc[e >> 2][e & 3], kNegLog2e, b_lo));
    } else if (mode == 1) {
      int64_t tq[16];  // element e: query 16 (e / 4) + 4 g + e % 4
      bwd_ts16<16>(tsq + 4 * g, tq);
#pragma unroll
      for (int e = 0; e < 16; ++e) put(e, __builtin_fmaf(sc[e >> 2][e & 3], kNegLog2e, tq[e] >= tcut ? b_hi : b_lo));
    } else if (small) {
      pairs(std::true_type{});
    } else {
      pairs(std::false_type{});
    }
    // dV^T += dO^T a and dK^T += Q^T dS, one 32-query half at a time: a
    // lane's elements 8 c .. 8 c + 7 are that half's k values in kv_col_frag's
    // order
    const bf16x8 fa0 = bwd_frag<T>(pa), fa1 = bwd_frag<T>(pa + 8);
    const bf16x8 fd0 = bwd_frag<T>(pd), fd1 = bwd_frag<T>(pd + 8);
    // step t: half c = t / (FV + FQ); dV tile ft, then dK tile ft
    constexpr int FV = DV / 16, FQ = DQK / 16;
    bwd_piped<2 * (FV + FQ), 4>(
        [&](int t) __attribute__((always_inline)) {
          const int c = t / (FV + FQ), u = t % (FV + FQ);
          return u < FV ? kv_col_frag<DV>(Os + 32 * c * DV + cov[u]) : kv_col_frag<DQK>(Qs + 32 * c * DQK + coq[u - FV]);
        },
        [&](int t, const bf16x8& x) __attribute__((always_inline)) {
          const int c = t / (FV + FQ), u = t % (FV + FQ);
          if (u < FV)
            dv[u] = mma16(x, c ? fa1 : fa0, dv[u]);
          else
            dk[u - FV] = mma16(x, c ? fd1 : fd0, dk[u - FV]);
        });
  };
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block 0 have landed
  __syncthreads();                // ... and every wave's, plus the tables
  for (int blk = 0; blk < nblk; blk += 2) {
    if (blk + 1 < nblk) issue(blk + 1, 1);
    consume(blk, 0);
    if (blk + 1 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (blk + 2 < nblk) issue(blk + 2, 0);
    consume(blk + 1, 1);
    if (blk + 2 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (kvalid) {
    const int64_t dvd = (s0 + jk) * (int64_t)a.N1 + K2 + h * DV + 4 * g;
    const int64_t dkd = (s0 + jk) * (int64_t)a.N1 + 2 * K2 + H * DQK + h * DQK + 4 * g;
    const float fv = kNegLn2 * inv_n;
#pragma unroll
    for (int ft = 0; ft < DV / 16; ++ft)
      bwd_out4<T, PRE>(a, dvd + 16 * ft, fv * dv[ft][0], fv * dv[ft][1], fv * dv[ft][2], fv * dv[ft][3]);
#pragma unroll
    for (int ft = 0; ft < DQK / 16; ++ft)
      bwd_out4<T, PRE>(a, dkd + 16 * ft, inv_n * dk[ft][0], inv_n * dk[ft][1], inv_n * dk[ft][2], inv_n * dk[ft][3]);
  }
}

// Bias-table gradients: column sums of the dq kernel's partial rows, per
// head (rows item * H + h); a table with head stride 0 sums every head (into
// head 0's row).  One workgroup per 64 result columns; its 16 waves take
// every 16th row each (four running sums apiece, so four loads are in
// flight), then the 16 partial sums are added in wave order: a fixed order,
// so the result is reproducible.
constexpr int kTabGroups = 16;
__global__ __launch_bounds__(64 * kTabGroups) void table_grad_kernel(const float* __restrict__ part, int64_t items,
                                                                     int H, int P, int NB, int pos_shared,
                                                                     int time_shared, float* __restrict__ gpos,
                                                                     float* __restrict__ gtime) {
  __shared__ float red[kTabGroups][64];
  const int W = P + NB;
  const int t = threadIdx.x, col = t & 63, g = t >> 6;
  const int c = blockIdx.x * 64 + col;  // column of the [H][P + NB] result
  const bool live = c < H * W;
  const int h = live ? c / W : 0, idx = live ? c - h * W : 0;
  const bool is_pos = idx < P;
  const bool sh = is_pos ? pos_shared : time_shared;
  // rows summed: every row (shared table, head 0) or rows it * H + h
  const int64_t nrows = !live || (sh && h > 0) ? 0 : (sh ? items * H : items);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int64_t k = g;
  for (; k + 3 * kTabGroups < nrows; k += 4 * kTabGroups) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t r = k + u * kTabGroups;
      acc[u] += part[(sh ? r : r * H + h) * W + idx];
    }
  }
#pragma unroll
  for (int u = 0; u < 3; ++u) {  // at most three rows left for this wave
    const int64_t r = k + u * kTabGroups;
    if (r < nrows) acc[u] += part[(sh ? r : r * H + h) * W + idx];
  }
  red[g][col] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (g != 0 || nrows == 0) return;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kTabGroups; ++i) sum += red[i][col];
  if (is_pos)
    gpos[(sh ? 0 : h) * P + idx] = sum;
  else
    gtime[(sh ? 0 : h) * NB + idx - P] = sum;
}

template <typename T, int DQK, int DV, bool PRE>
static hipError_t bwd_dims_pre(const BwdArgs& a, int64_t grid, hipStream_t s) {
  const size_t sh_dq = (size_t)5 * (a.P + a.NB) * sizeof(float), sh_kv = (size_t)(a.P + a.NB) * sizeof(float);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV, PRE>), dim3((unsigned)grid), dim3(256), sh_dq, s, a);
  if constexpr (std::is_same<T, bf16>::value) {
    // two 64-key halves per work item
    hipLaunchKernelGGL((attn_bwd_kv16_kernel<DQK, DV, PRE>), dim3((unsigned)(2 * grid)), dim3(256), sh_kv, s, a);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, DQK, DV, false, PRE>), dim3((unsigned)grid), dim3(256), sh_kv, s, a);
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, DQK, DV, true, PRE>), dim3((unsigned)grid), dim3(256), sh_kv, s, a);
  }
  return hipGetLastError();
}

template <typename T, int DQK, int DV>
static hipError_t bwd_dims(const BwdArgs& a, int64_t grid, hipStream_t s) {
  return a.pre ? bwd_dims_pre<T, DQK, DV, true>(a, grid, s) : bwd_dims_pre<T, DQK, DV, false>(a, grid, s);
}

hipError_t launch_attn_bwd(const hstu_desc& d, const int64_t* off, const int32_t* ncand, int32_t B, int64_t T,
                           const int64_t* ts, const hstu_bias_tables& tab, const void* q, const void* k,
                           const void* v, const void* dout, float* dact, const void* pre, void* dpre,
                           float* tab_part, float* gpos, float* gtime, const AttnScratch& sc, hipStream_t s) {
  if (T == 0) return hipSuccess;
  BwdArgs a;
  a.off = off;
  a.ncand = ncand;
  a.ts = ts;
  a.pos_tab = tab.pos;
  a.time_tab = tab.time;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.dact = dact;
  a.pre = pre;
  a.dpre = dpre;
  a.tab_part = tab_part;
  a.tiles = sc.tiles;
  a.tbase = sc.tbase;
  a.counts = sc.counts;
  a.tstat = sc.tstat;
  a.T = T;
  a.H = d.num_heads;
  a.P = d.pos_buckets;
  a.NB = d.time_buckets;
  a.sbits = d.time_sub_bits;
  a.pos_stride = tab.pos_head_stride;
  a.time_stride = tab.time_head_stride;
  a.norm_len = d.norm_len;
  a.shared_pos = (d.flags & HSTU_CAND_SHARED_POS) ? 1 : 0;
  a.N1 = 2 * d.num_heads * (d.dqk + d.dv);
  const int64_t items = attn_max_tiles(T, B);
  const int64_t grid = items * d.num_heads;
  hipError_t e = hipErrorInvalidValue;
#define HSTU_BWD_CASE(TT, Q, V_) \
  else if (d.dqk == Q && d.dv == V_) e = bwd_dims<TT, Q, V_>(a, grid, s);
  if (d.dtype == HSTU_BF16) {
    if (false) {
    }
    HSTU_BWD_CASE(bf16, 32, 32)
    HSTU_BWD_CASE(bf16, 64, 64)
    HSTU_BWD_CASE(bf16, 128, 128)
  } else {
    if (false) {
    }
    HSTU_BWD_CASE(float, 32, 32)
    HSTU_BWD_CASE(float, 64, 64)
  }
#undef HSTU_BWD_CASE
  if (e != hipSuccess) return e;
  const int W = d.pos_buckets + d.time_buckets;
  hipLaunchKernelGGL(table_grad_kernel, dim3((unsigned)((d.num_heads * W + 63) / 64)), dim3(64 * kTabGroups), 0, s, tab_part,
                     items, (int)d.num_heads, (int)d.pos_buckets, (int)d.time_buckets,
                     tab.pos_head_stride == 0 ? 1 : 0, tab.time_head_stride == 0 ? 1 : 0, gpos, gtime);
  return hipGetLastError();
}

}  // namespace hstu
