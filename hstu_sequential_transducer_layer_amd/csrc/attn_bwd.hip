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
// Tiles in LDS are plain row-major rows padded by 16 bytes.
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
  float* tab_part;    // [gridDim.x][P + NB]: per-workgroup bias-table gradients (dq kernel)
  const int2* tiles;
  const int32_t* counts;
  int64_t T;
  int H, P, NB, sbits, pos_stride, time_stride, norm_len, shared_pos, N1;
};

// Rows of 64 x D in LDS, row stride D + 16 bytes.
template <typename T, int D>
struct BTile {
  static constexpr int V = Elem<T>::kVec, CPR = D / V, LD = D + V;
};

// 64 rows of D elements from src (row r at src + r * stride) into a padded
// tile; rows at or past `avail` (>= 1) repeat row avail - 1.
template <typename T, int D>
__device__ __forceinline__ void bwd_copy(const T* __restrict__ src, int64_t stride, int avail, T* lds) {
  typedef BTile<T, D> Bt;
  for (int ch = threadIdx.x; ch < 64 * Bt::CPR; ch += 256) {
    const int r = ch / Bt::CPR, c = ch - r * Bt::CPR;
    const int rr = min(r, avail - 1);
    st16(lds + r * Bt::LD + c * Bt::V, ld16(src + rr * stride + c * Bt::V));
  }
}

// A operand from tile rows: row r, elements e0 .. e0 + 7.
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::Frag bwd_row_frag(const T* lds, int r, int e0) {
  typedef typename Elem<T>::Frag Frag;
  const T* p = lds + r * BTile<T, D>::LD + e0;
  if constexpr (Elem<T>::kVec == 8) {
    return *reinterpret_cast<const Frag*>(p);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
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
  typename Elem<T>::Frag x;
  const int half = lane >> 5;
  if constexpr (Elem<T>::kVec == 8) {
    const int a = lane & 15;
    const int row = kb + 4 * half + (a >> 2);
    const int col = 32 * nt + 16 * ((lane >> 4) & 1) + 4 * (a & 3);
    const bwd_v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(lds + row * BTile<T, D>::LD + col));
    const bwd_v4i16 x1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((bwd_lds_v4i16*)(lds + (row + 8) * BTile<T, D>::LD + col));
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
    for (int e = 0; e < 8; ++e) x[e] = lds[(kb + 8 * (e >> 2) + 4 * half + (e & 3)) * BTile<T, D>::LD + f];
  }
  return x;
}

// Min and max of 64 int64 values held one per lane (wave 0 of a block copy).
__device__ __forceinline__ void bwd_minmax64(int64_t v, int64_t& mn, int64_t& mx) {
  mn = v;
  mx = v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t a = __shfl_xor(mn, o, kWave), b = __shfl_xor(mx, o, kWave);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
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

template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  typedef typename Elem<T>::Frag Frag;
  __shared__ __attribute__((aligned(16))) T Ks[64 * BTile<T, DQK>::LD];
  __shared__ __attribute__((aligned(16))) T Vs[64 * BTile<T, DV>::LD];
  __shared__ int64_t tsk[64];
  __shared__ int64_t kmm[2];  // the block's earliest and latest key timestamp
  // pos[P], time[NB], then one gradient histogram [P + NB] per wave (a
  // wave's updates land in program and lane order, so the sums are
  // reproducible; the four are added in wave order at the end)
  extern __shared__ float tabs[];
  const int H = a.H, h = blockIdx.x % H, item = blockIdx.x / H;
  const int P = a.P, NB = a.NB;
  float* pos_s = tabs;
  float* time_s = tabs + P;
  const int tid = threadIdx.x;
  float* part = a.tab_part + (int64_t)blockIdx.x * (P + NB);
  if (item >= a.counts[0]) {  // whole workgroup: an empty partial row
    for (int i = tid; i < P + NB; i += 256) part[i] = 0.f;
    return;
  }
  for (int i = tid; i < P; i += 256)
    pos_s[i] = to_f32(reinterpret_cast<const T*>(a.pos_tab)[(int64_t)h * a.pos_stride + i]);
  for (int i = tid; i < NB; i += 256)
    time_s[i] = to_f32(reinterpret_cast<const T*>(a.time_tab)[(int64_t)h * a.time_stride + i]);
  for (int i = tid; i < 4 * (P + NB); i += 256) tabs[P + NB + i] = 0.f;
  float* gpos = tabs + (P + NB) * (1 + wave_id());
  float* gtime = gpos + P;
  const int2 tl = a.tiles[item];
  const SeqInfo si = seq_info(a.off, a.ncand, tl.x, a.T);
  const int L = si.len, nh = si.nhist;
  const int64_t s0 = si.start;
  const int i0 = tl.y * 128, iend = min(i0 + 128, L);
  const int lane = tid & 63, w = wave_id(), l32 = lane & 31, half = lane >> 5;
  const int r0 = i0 + 32 * w, iq = r0 + l32;
  const bool qvalid = iq < iend;
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
    if (qvalid) qf[c] = bwd_row_frag<T, DQK>(qrow - 0, 0, 16 * c + 8 * half);
  }
#pragma unroll
  for (int c = 0; c < DV / 16; ++c) {
    df[c] = Frag{};
    if (qvalid) df[c] = bwd_row_frag<T, DV>(drow, 0, 16 * c + 8 * half);
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
  for (int blk = 0; blk < nblk_a + nblk_b; ++blk) {
    const int j0 = blk < nblk_a ? blk * 64 : jb0 + (blk - nblk_a) * 64;
    __syncthreads();  // the previous block's reads are done
    bwd_copy<T, DQK>(kg + (int64_t)j0 * DQK, DQK, L - j0, Ks);
    bwd_copy<T, DV>(vg + (int64_t)j0 * DV, DV, L - j0, Vs);
    if (tid < 64) {
      const int64_t t = a.ts[s0 + min(j0 + tid, L - 1)];
      tsk[tid] = t;
      int64_t mn, mx;
      bwd_minmax64(t, mn, mx);
      if (tid == 0) {
        kmm[0] = mn;
        kmm[1] = mx;
      }
    }
    __syncthreads();
    if (r0 >= iend) continue;
    // A far block: every key a history key strictly before the wave's first
    // row and at least R positions from it (position bucket 2R, no mask);
    // with one time bucket per row over the block's time span, the bias is
    // one value per row (wave-uniform test).
    bool fast = j0 + 63 < L && j0 + 63 < nh && j0 + 63 < r0 && position(r0, nh, shared) - (j0 + 63) >= R;
    int bt_row = 0;
    float b_row = 0.f;
    if (fast) {
      const int lo = time_bucket(wrap_sub(ts_q, kmm[1]), NB, a.sbits);
      const int hi = time_bucket(wrap_sub(ts_q, kmm[0]), NB, a.sbits);
      fast = __all(lo == hi || !qvalid);
      bt_row = lo;
      b_row = pos_s[2 * R] + time_s[lo];
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x16 sc = f32x16{}, da = f32x16{};
#pragma unroll
      for (int c = 0; c < DQK / 16; ++c) sc = mma_k16(bwd_row_frag<T, DQK>(Ks, kh * 32 + l32, 16 * c + 8 * half), qf[c], sc);
#pragma unroll
      for (int c = 0; c < DV / 16; ++c) da = mma_k16(bwd_row_frag<T, DV>(Vs, kh * 32 + l32, 16 * c + 8 * half), df[c], da);
      float ds[16];
      if (fast) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sc[r] + b_row;
          const float sg = bwd_sigmoid(s);
          ds[r] = qvalid ? da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n : 0.f;
          sum += ds[r];
        }
        far_hi += sum;
        if (bt_row != run_bt) {
          if (run != 0.f) atomicAdd(&gtime[run_bt], run);
          run_bt = bt_row;
          run = 0.f;
        }
        run += sum;
      } else
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3), j = j0 + kl;
        const bool valid = qvalid && j < L && attends(iq, j, nh);
        const int bp = pos_bucket(p_q, position(j, nh, shared), R);
        const int bt = time_bucket(wrap_sub(ts_q, tsk[kl]), NB, a.sbits);
        const float s = sc[r] + pos_s[bp] + time_s[bt];
        const float sg = bwd_sigmoid(s);
        const float g = da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n;
        ds[r] = valid ? g : 0.f;
        if (valid) {
          if (bp == 0)
            far_lo += g;
          else if (bp == 2 * R)
            far_hi += g;
          else
            atomicAdd(&gpos[bp], g);
          if (bt != run_bt) {
            if (run != 0.f) atomicAdd(&gtime[run_bt], run);
            run_bt = bt;
            run = 0.f;
          }
          run += g;
        }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const Frag pf = bwd_frag<T>(ds + 8 * c2);
#pragma unroll
        for (int n = 0; n < DQK / 32; ++n)
          dq[n] = mma_k16(bwd_col_frag<T, DQK>(Ks, kh * 32 + 16 * c2, n, lane), pf, dq[n]);
      }
    }
  }
  if (qvalid) {
    float* dst = a.dact + (s0 + iq) * (int64_t)a.N1 + 2 * K2 + h * DQK;
#pragma unroll
    for (int n = 0; n < DQK / 32; ++n)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(dst + 32 * n + 8 * g4 + 4 * half) =
            make_float4(dq[n][4 * g4], dq[n][4 * g4 + 1], dq[n][4 * g4 + 2], dq[n][4 * g4 + 3]);
  }
  if (run != 0.f) atomicAdd(&gtime[run_bt], run);
  if (far_lo != 0.f) atomicAdd(&gpos[0], far_lo);
  if (far_hi != 0.f) atomicAdd(&gpos[2 * R], far_hi);
  __syncthreads();  // every LDS histogram update is done
  for (int i = tid; i < P + NB; i += 256) {
    const float* hw = tabs + (P + NB) + i;
    part[i] = ((hw[0] + hw[P + NB]) + hw[2 * (P + NB)]) + hw[3 * (P + NB)];
  }
}

template <typename T, int DQK, int DV, bool DK>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_kernel(BwdArgs a) {
  typedef typename Elem<T>::Frag Frag;
  constexpr int DACC = DK ? DQK : DV;  // width of this pass's gradient
  __shared__ __attribute__((aligned(16))) T Qs[64 * BTile<T, DQK>::LD];
  __shared__ __attribute__((aligned(16))) T Os[64 * BTile<T, DV>::LD];
  __shared__ int64_t tsq[64];
  __shared__ int64_t qmm[2];  // the block's earliest and latest query timestamp
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
    if (kvalid) kf[c] = bwd_row_frag<T, DQK>(krow, 0, 16 * c + 8 * half);
  }
  if (DK) {
#pragma unroll
    for (int c = 0; c < DV / 16; ++c) {
      vf[c] = Frag{};
      if (kvalid) vf[c] = bwd_row_frag<T, DV>(vrow, 0, 16 * c + 8 * half);
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
  for (int i0 = qb0; i0 < qend; i0 += 64) {
    __syncthreads();
    bwd_copy<T, DQK>(qg + (int64_t)i0 * DQK, DQK, L - i0, Qs);
    bwd_copy<T, DV>(og + (int64_t)i0 * K2, K2, L - i0, Os);
    if (tid < 64) {
      const int64_t t = a.ts[s0 + min(i0 + tid, L - 1)];
      tsq[tid] = t;
      int64_t mn, mx;
      bwd_minmax64(t, mn, mx);
      if (tid == 0) {
        qmm[0] = mn;
        qmm[1] = mx;
      }
    }
    __syncthreads();
    if (kr0 >= jend) continue;
    // A far block (the dq kernel's test with queries and keys swapped): all
    // the wave's keys history keys strictly before the block's first query
    // and at least R positions from it; one time bucket per key.
    const int k_last = min(kr0 + 31, jend - 1);
    bool fast = i0 + 63 < L && k_last < nh && i0 > k_last && position(i0, nh, shared) - k_last >= R;
    float b_key = 0.f;
    if (fast) {
      const int lo = time_bucket(wrap_sub(qmm[0], ts_k), NB, a.sbits);
      const int hi = time_bucket(wrap_sub(qmm[1], ts_k), NB, a.sbits);
      fast = __all(lo == hi || !kvalid);
      b_key = pos_s[2 * R] + time_s[lo];
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
      if (fast) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float s = sc[r] + b_key;
          const float sg = bwd_sigmoid(s);
          const float val = DK ? da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n : s * sg * inv_n;
          g[r] = kvalid ? val : 0.f;
        }
      } else
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qh * 32 + 8 * (r >> 2) + 4 * half + (r & 3), i = i0 + ql;
        const bool valid = kvalid && i < L && attends(i, jk, nh);
        const int bp = pos_bucket(position(i, nh, shared), p_k, R);
        const int bt = time_bucket(wrap_sub(tsq[ql], ts_k), NB, a.sbits);
        const float s = sc[r] + pos_s[bp] + time_s[bt];
        const float sg = bwd_sigmoid(s);
        const float val = DK ? da[r] * sg * (1.0f + s * (1.0f - sg)) * inv_n : s * sg * inv_n;
        g[r] = valid ? val : 0.f;
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
  }
  if (kvalid) {
    float* dst = a.dact + (s0 + jk) * (int64_t)a.N1 + (DK ? 2 * K2 + H * DQK + h * DQK : K2 + h * DV);
#pragma unroll
    for (int n = 0; n < DACC / 32; ++n)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(dst + 32 * n + 8 * g4 + 4 * half) =
            make_float4(acc[n][4 * g4], acc[n][4 * g4 + 1], acc[n][4 * g4 + 2], acc[n][4 * g4 + 3]);
  }
}

// Bias-table gradients: column sums of the dq kernel's partial rows, per
// head (rows item * H + h); a table with head stride 0 sums every head.
__global__ __launch_bounds__(256) void table_grad_kernel(const float* __restrict__ part, int64_t items, int H, int P,
                                                         int NB, int pos_shared, int time_shared,
                                                         float* __restrict__ gpos, float* __restrict__ gtime) {
  const int W = P + NB;
  const int c = blockIdx.x * 256 + threadIdx.x;  // column of the [H][P + NB] result
  if (c >= H * W) return;
  const int h = c / W, idx = c - h * W;
  const bool is_pos = idx < P;
  const bool sh = is_pos ? pos_shared : time_shared;
  if (sh && h > 0) return;  // head 0 sums all heads
  float s = 0.f;
  for (int hh = sh ? 0 : h; hh < (sh ? H : h + 1); ++hh)
    for (int64_t it = 0; it < items; ++it) s += part[(it * H + hh) * W + idx];
  if (is_pos)
    gpos[(sh ? 0 : h) * P + idx] = s;
  else
    gtime[(sh ? 0 : h) * NB + idx - P] = s;
}

template <typename T, int DQK, int DV>
static hipError_t bwd_dims(const BwdArgs& a, int64_t grid, hipStream_t s) {
  const size_t sh_dq = (size_t)5 * (a.P + a.NB) * sizeof(float), sh_kv = (size_t)(a.P + a.NB) * sizeof(float);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV>), dim3((unsigned)grid), dim3(256), sh_dq, s, a);
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, DQK, DV, false>), dim3((unsigned)grid), dim3(256), sh_kv, s, a);
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, DQK, DV, true>), dim3((unsigned)grid), dim3(256), sh_kv, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const hstu_desc& d, const int64_t* off, const int32_t* ncand, int32_t B, int64_t T,
                           const int64_t* ts, const hstu_bias_tables& tab, const void* q, const void* k,
                           const void* v, const void* dout, float* dact, float* tab_part, float* gpos,
                           float* gtime, const AttnScratch& sc, hipStream_t s) {
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
  a.tab_part = tab_part;
  a.tiles = sc.tiles;
  a.counts = sc.counts;
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
  hipLaunchKernelGGL(table_grad_kernel, dim3((unsigned)((d.num_heads * W + 255) / 256)), dim3(256), 0, s, tab_part,
                     items, (int)d.num_heads, (int)d.pos_buckets, (int)d.time_buckets,
                     tab.pos_head_stride == 0 ? 1 : 0, tab.time_head_stride == 0 ? 1 : 0, gpos, gtime);
  return hipGetLastError();
}

}  // namespace hstu
