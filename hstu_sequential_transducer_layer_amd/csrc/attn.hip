// Stage 2: pointwise aggregated attention over jagged sequences.
//
//   AV_i^h = (1/N_b) sum_j M_ij SiLU(q_i.k_j + pos[h][bp(i,j)] + time[h][bt(i,j)]) v_j
//
// Sources: page "4.4 Scaling Recommendation Models", section "Generative
// Recommenders and HSTU" (second layer equation; SiLU applied to each score on
// its own with a constant normaliser such as the sequence length; bias on
// position and time difference; candidates appended to the history that see
// the history but not one another) and section "Code" (per-head bias added to
// q.k, lower-triangular mask keeping the diagonal, division by n, no softmax
// and no 1/sqrt(d)); page "HSTU: The First Exploration of the Scaling Law",
// 7.1.4 Innovations 1-2 and 7.1.5 M-FALCON layer 1.
//
// Work item: (sequence b, 128-row query tile, head h), one workgroup of four
// waves, each wave owning 32 query rows.  The key range is streamed in 64-key
// blocks through LDS: the history keys up to the tile's last row, then (for
// candidate rows) the block(s) holding the candidates' own diagonal.  Nothing
// is renormalised across blocks — pointwise weights just add — so there is no
// running max or rescaling, and blocks no row of a wave can attend are skipped.
//
// Per key block, per wave:
//   S^T[key, query] = K_blk . Q^T        MFMA, A = K rows from LDS, B = Q in registers
//   P = mask * SiLU(S^T + biases)        registers (lane = query, 16 keys)
//   O^T[dv, query] += V^T_blk . P^T      MFMA, A = V^T from LDS, B = P straight
//                                        from the S^T accumulators
// The S^T accumulator of lane l holds keys 8*(r/4) + 4*(l/32) + (r%4); those
// eight keys per k16 step are used as that MFMA's k-order for both operands,
// so P never leaves registers.  V is transposed into LDS while staged.
//
// Output: AV minus its per-(row, head) mean over dv, in the layer dtype, plus
// fp32 (mean, sum of squared deviations) per (row, head) for the LayerNorm.
#include "common.h"
#include "kernels.h"

namespace hstu {

// Entries of padding on each side of the position-bias table in LDS (edge
// values repeated): mode 2 reads p(i) - j in [-94, R + 94) without a clamp.
constexpr int kPosPad = 96;

template <typename T, int DQK, int DV>
struct AttnCfg {
  static constexpr int BM = kAttnBM, BN = kAttnBN, NW = BM / 32;
  static constexpr int NT = NW * kWave;
  static constexpr int V = Elem<T>::kVec;                  // elements per 16-byte chunk
  static constexpr int KCPR = DQK / V, VCPR = DV / V;      // chunks per K / V row
  static constexpr int KCH = BN * KCPR, VCH = BN * VCPR;   // chunks per block
  static_assert(KCH % NT == 0 && VCH % NT == 0, "block chunks must split evenly over waves");
};

// LDS tiles are written by direct global->LDS loads, 16 bytes per lane in
// lane order, so rows cannot be padded; instead chunk c of row r is stored at
// chunk c ^ swz(r).  The LDS has 64 four-byte banks (16 chunk slots of 16
// bytes per 256-byte line).  K rows (CPR chunks) are read 16 bytes per lane
// down 16 consecutive rows: k_swz spreads those rows over all 16 slots.  V
// rows are read through the transposing 8-byte read, 4 consecutive rows x 4
// consecutive chunks per 32 lanes: v_swz spreads those 16 pieces likewise.
template <int CPR>
__device__ __forceinline__ int k_swz(int r) {
  return CPR >= 16 ? (r & 15) & (CPR - 1) : ((r / (16 / CPR)) & (CPR - 1));
}
template <int CPR>
__device__ __forceinline__ int v_swz(int r) {
  return CPR >= 16 ? 4 * (r & 3) : (CPR == 8 ? 4 * ((r >> 1) & 1) : 0);
}

struct AttnArgs {
  const int64_t* off;      // query rows of each sequence
  const int32_t* ncand;
  const int64_t* ts;       // query rows' timestamps
  const int64_t* koff;     // key rows of each sequence (= off unless cached)
  const int64_t* kts;      // key rows' timestamps
  const int32_t* mtotal;   // cached: each sequence's full candidate count
  const void* pos_tab;
  const void* time_tab;
  const void* q;
  const void* k;           // key rows' K, V  [H, TK, d]
  const void* v;
  const void* qk;          // cached: the query rows' own K, V [H, T, d]
  const void* qv;
  void* av;
  float* stats;
  float* part;             // cached: per-chunk partial AV [kCandMaxSplit][T][H * DV]
  const int32_t* nsplit;   // cached: history chunks per sequence
  const uint8_t* qtypes;   // typed: query rows' token types
  const int32_t* kty;      // typed: key rows' token types (int32, clamped)
  const void* type_tab;    // typed: [NT][NT] per head
  int NT, type_stride;
  const int2* tiles;
  const int32_t* counts;   // [0]: work items
  const int32_t* rel;      // per key row: offset from its key block's earliest timestamp
  const int64_t* tstat;    // per key block's first row: earliest, latest timestamp
  float* dump;             // inspection: [H][dump_slots][dump_len] biases
  const int32_t* dump_slot;  // inspection: per query row its slot, or -1
  int dump_slots, dump_len;
  int64_t T, TK;           // query rows, key rows
  int H, P, NB, sbits, pos_stride, time_stride, norm_len, shared_pos;
};

template <typename T>
struct LdsPtr {
  typedef __attribute__((address_space(3))) T type;
};
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Asynchronous copy of one key block of a [rows, D] head-major tensor into a
// swizzled LDS tile: every wave issues PER 16-byte-per-lane direct loads.
// Load i of wave w fills the 64 / CPR rows starting at (i * NW + w) * 64 / CPR,
// so a lane's rows in successive loads lie STRIDE rows apart, a multiple of
// the swizzle period (16 rows): its source offset is one fixed value plus
// i * STRIDE rows.  Each load is then a wave-uniform base (scalar registers)
// plus that fixed per-lane offset.  In a block that runs past the sequence's
// end, rows past it read the sequence's last row instead (finite values that
// the mask turns into zero weight), so no other sequence's data is read.
template <typename T, int D, int NW, int CPR, bool IS_K>
struct TileCopy {
  static constexpr int V = Elem<T>::kVec;
  static constexpr int PER = 64 * CPR / (NW * 64);  // BN = 64 rows
  static constexpr int STRIDE = NW * 64 / CPR;      // rows between a lane's loads
  static constexpr int LOG_D = D == 32 ? 5 : D == 64 ? 6 : 7;
  static_assert(D == 32 || D == 64 || D == 128, "head width");
  static_assert(PER == 1 || STRIDE % 16 == 0, "loads must share the swizzle");
  int r0;    // this lane's row in load 0
  int off0;  // its source offset (elements) in load 0
  __device__ __forceinline__ void init(int w, int lane) {
    const int slot = w * 64 + lane;
    const int pc = slot % CPR;
    r0 = slot / CPR;
    off0 = r0 * D + (pc ^ (IS_K ? k_swz<CPR>(r0) : v_swz<CPR>(r0))) * V;
  }
  // g: the block's first row; rows: rows of the sequence from there (>= 1).
  __device__ __forceinline__ void issue(const T* __restrict__ g, int rows, T* lds, int w) const {
    const uint32_t lane_bytes = (uint32_t)off0 * (uint32_t)sizeof(T);
    if (rows >= 64) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        __builtin_amdgcn_global_load_lds(
            (glb_void*)(reinterpret_cast<const char*>(g + i * STRIDE * D) + lane_bytes),
            (lds_void*)(lds + (i * NW + w) * 64 * V), 16, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int r = r0 + i * STRIDE, rr = min(r, rows - 1);
        __builtin_amdgcn_global_load_lds((glb_void*)(g + off0 + i * STRIDE * D + (rr - r) * D),
                                         (lds_void*)(lds + (i * NW + w) * 64 * V), 16, 0, 0);
      }
    }
  }
};

// A operand of S^T (K rows): row `r`, 8 elements starting at element `e0`.
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::Frag k_frag(const T* lds, int r, int e0) {
  constexpr int V = Elem<T>::kVec, CPR = D / V;
  typedef typename Elem<T>::Frag Frag;
  if constexpr (V == 8) {
    return *reinterpret_cast<const Frag*>(lds + r * D + ((e0 / V) ^ k_swz<CPR>(r)) * V);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(lds + r * D + ((e0 / V) ^ k_swz<CPR>(r)) * V);
    const f32x4 b = *reinterpret_cast<const f32x4*>(lds + r * D + ((e0 / V + 1) ^ k_swz<CPR>(r)) * V);
    return Frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// A operand of O^T (V^T): for this lane's value column n = 32*nt + (lane%32)
// the eight keys kb + 4*(lane/32) + {0,1,2,3} and kb + 8 + 4*(lane/32) + {0..3}.
// bf16: two transposing LDS reads; each 16-lane group of a ds_read_b64_tr_b16
// returns, to lane l, element l%4 of the 4-element pieces addressed by lanes
// l/4, 4+l/4, 8+l/4, 12+l/4; so source lane a of the group addresses row
// k0 + a/4, columns D + 4*(a%4) .. +3.
template <typename T, int DV>
__device__ __forceinline__ typename Elem<T>::Frag v_frag(const T* lds, int kb, int nt, int lane) {
  constexpr int V = Elem<T>::kVec, CPR = DV / V;
  if constexpr (V == 8) {
    const int a = lane & 15;
    const int row = kb + 4 * (lane >> 5) + (a >> 2);
    const int col = 32 * nt + 16 * ((lane >> 4) & 1) + 4 * (a & 3);
    const int c = col / V, off = col % V;
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(lds + row * DV + (c ^ v_swz<CPR>(row)) * V + off));
    const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16*)(lds + (row + 8) * DV + (c ^ v_swz<CPR>(row + 8)) * V + off));
    bf16x8 f;
    const bf16* p0 = reinterpret_cast<const bf16*>(&x0);
    const bf16* p1 = reinterpret_cast<const bf16*>(&x1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = p0[e];
      f[4 + e] = p1[e];
    }
    return f;
  } else {
    const int n = 32 * nt + (lane & 31), k0 = kb + 4 * (lane >> 5);
    const int c = n / V, off = n % V;
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = k0 + (e >> 2) * 8 + (e & 3);
      f[e] = lds[row * DV + (c ^ v_swz<CPR>(row)) * V + off];
    }
    return f;
  }
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::Frag to_frag(const float* p);
template <>
__device__ __forceinline__ bf16x8 to_frag<bf16>(const float* p) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (bf16)p[e];
  return f;
}
template <>
__device__ __forceinline__ f32x8 to_frag<float>(const float* p) {
  f32x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = p[e];
  return f;
}

// bucket_floor for buckets reached by dt < 2^24 (k < 24), in 32 bits and
// with selects only.
__device__ __forceinline__ int bucket_floor_small(int b, int s) {
  const int c = b - 1, k = min(c >> s, 30), sub = c & ((1 << s) - 1);
  const int sh = s - k;  // > 0 only when k < s (then sh <= s <= 4)
  const int ge = (1 << k) | (sub << (k >= s ? k - s : 0));
  const int lt = (1 << k) + ((sub + (1 << (sh > 0 ? sh : 0)) - 1) >> (sh > 0 ? sh : 0));
  return k >= s ? ge : lt;
}

// Per-(wave, key block) inputs of the score -> weight step.  Lane offsets are
// folded into the per-lane fields, so the key index of accumulator entry r of
// half kh is a compile-time constant c = 32 kh + 8 (r / 4) + r % 4 plus jq.
struct ElemCtx {
  int jq;        // j0 + 4 * (lane / 32): key index of c = 0
  int iq, nh, p_q, R, NB, sbits, L;
  SmallBucket bk;
  bool shared;
  float c_lo, c_hi;
  int32_t thr;   // MODE 1: keys with offset <= thr take c_hi
  int32_t hi32;  // MODES 2, 4: t_i - (block's earliest timestamp)
  int pq0, iq0;  // MODE 2: p(i) - jq and i - jq
  const float* posb;  // MODE 2: &pos_s[R + p(i) - jq - 63]; key jq + c reads posb[63 - c]
  float cpos_far;     // MODE 4: the position bias of every pair
  int64_t ts_q;
  const float* pos_s;
  const float* time_s;
  int rel_off;           // MODES 1, 2: jq - j0, the index of key jq in the block's offsets
  const int64_t* ts;     // MODE 3: the sequence's timestamps (global)
};

// Scores -> pointwise weights for one 32-key half (kb = 32 kh) held by this
// lane: query iq, keys jq + kb + 8 (r / 4) + r % 4.  Every variant is
// branch-free.
//   MODE 0: every pair attended, one bias per row (c_lo: time bucket and
//           position bias both constant over the block).
//   MODE 1: every pair attended, bias c_hi for keys whose offset from the
//           block's earliest timestamp is <= thr, else c_lo.
//   MODE 2: a block of history keys only, near the wave's rows: time
//           bucket, relative-position bias and causal mask per pair, with
//           t_i - t_j = hi32 - offset_j in 32 bits (|dt| < 2^24 over the
//           block) and position(j) = j.  Here p(i) - j lies in [-94, R + 94)
//           (the block is active for the wave and not R positions away), so
//           the position bias is read without a clamp from the table padded
//           with its edge values, at a per-lane base plus a constant offset.
//   MODE 3: any block: the same from the 64-bit timestamps, with shared
//           candidate positions and the candidate mask.
//   MODE 4: a full block of history keys at least R positions from every
//           row whose rows span three or more time buckets: time bucket per
//           pair as in mode 2, constant position bias, no mask.
// The bias (times -log2 e) of the pair (query iq, key jq + c) in weight mode
// MODE, and whether the pair is attended; rel is the key's time offset from
// its block's earliest timestamp (modes 1 and 2).
template <int MODE>
__device__ __forceinline__ float elem_bias(const ElemCtx& x, int c, int32_t rel, bool& att) {
  att = true;
  if (MODE == 0) return x.c_lo;
  if (MODE == 1) return rel <= x.thr ? x.c_hi : x.c_lo;
  if (MODE == 2) {
    const int bt = time_bucket_med3((int)((uint32_t)x.hi32 - (uint32_t)rel), x.bk);
    att = c <= x.iq0;  // j <= i
    return x.time_s[bt] + x.posb[63 - c];
  }
  if (MODE == 4) return x.time_s[time_bucket_med3((int)((uint32_t)x.hi32 - (uint32_t)rel), x.bk)] + x.cpos_far;
  const int j = x.jq + c;
  att = attends(x.iq, j, x.nh);
  return x.time_s[time_bucket(wrap_sub(x.ts_q, x.ts[min(j, x.L - 1)]), x.NB, x.sbits)] +
         x.pos_s[pos_bucket(x.p_q, position(j, x.nh, x.shared), x.R)];
}

// The time offsets of keys kb + 8 g + 0..3 (modes 1, 2 and 4; zeros otherwise)
// out of the block's offsets rb in LDS.  rb is passed down from the LDS
// array itself, never through a merged or stored pointer: the compiler can
// then tell these reads from a global->LDS copy in flight into the other
// buffer, and does not wait for that copy before them.
template <int MODE>
__device__ __forceinline__ void elem_rel4(const ElemCtx& x, const int32_t* rb, int kb, int g, int32_t (&rel)[4]) {
  if (MODE == 1 || MODE == 2 || MODE == 4) {
    const int4 rv = *reinterpret_cast<const int4*>(rb + x.rel_off + kb + 8 * g);
    rel[0] = rv.x; rel[1] = rv.y; rel[2] = rv.z; rel[3] = rv.w;
  } else {
    rel[0] = rel[1] = rel[2] = rel[3] = 0;
  }
}

template <int MODE>
__device__ __forceinline__ void elems(const f32x16& s, float (&p)[16], int kb, const ElemCtx& x,
                                      const int32_t* rb) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    int32_t rel[4];
    elem_rel4<MODE>(x, rb, kb, g, rel);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e, c = kb + 8 * g + e;
      bool att;
      const float b = elem_bias<MODE>(x, c, rel[e], att);
      const float v = silu_neglog2e(s[r], b);
      p[r] = att ? v : 0.f;
    }
  }
}

// Inspection: the biases of this lane's row for both 32-key halves of the
// block, written at dst[j] for keys j < L (NaN where the pair is masked).
template <int MODE>
__device__ __forceinline__ void dump_block(const ElemCtx& x, const int32_t* rb, float* dst, int L) {
#pragma unroll
  for (int kb = 0; kb < 64; kb += 32)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      int32_t rel[4];
      elem_rel4<MODE>(x, rb, kb, g, rel);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = kb + 8 * g + e, j = x.jq + c;
        bool att;
        const float b = elem_bias<MODE>(x, c, rel[e], att);
        if (j < L) dst[j] = att ? b : __builtin_nanf("");
      }
    }
}

// Facts about this lane's query row and its wave that the per-block
// classification needs.
struct QueryRow {
  int r0, rlast, iq, p_q, pmin_q;  // wave's first / last row, this row, positions
  bool qvalid;
  int64_t ts_q;
  int32_t rq;   // ts_q - t0 when every row of the wave is within 2^29 of t0 (narrow)
  bool narrow;  // wave-uniform
  uint64_t idle;  // lanes without a query row (they take no part in the wave's tests)
};

// Per-(workgroup) constants of the classification.
struct SeqCtx {
  int L, nh, R, NB, sbits;
  SmallBucket bk;  // the small-range bucket's clamp bounds and shift
  bool shared;
  float cpos_far;  // bias of every pair at relative distance >= R
  const float* pos_s;
  const float* time_s;
  const int64_t* ts;  // the sequence's timestamps
  int64_t t0;         // reference time of the 32-bit classification: the first key's
};

// Whether any row of the wave (which has rows) attends a key of the block
// starting at j0.
__device__ __forceinline__ bool block_active(int j0, const QueryRow& q, const SeqCtx& sq) {
  const bool any_hist = j0 < sq.nh && j0 <= q.rlast;
  const bool any_self = max(max(q.r0, sq.nh), j0) <= min(q.rlast, j0 + kAttnBN - 1);
  return any_hist || any_self;
}

// Weight mode of one (wave, key block) — wave-uniform — and the per-lane
// context of the weight step.  Per query row the block's time differences lie
// in [lo, hi]; the bucket is monotone in dt, so one bucket, or two split by a
// threshold on the key's time offset, covers the whole row.
//
// When the block's and the wave's timestamps all lie within 2^29 of the
// reference t0 (the usual case; a wave-uniform test on scalars, differences
// modulo 2^64), the row's range comes from 32-bit differences of times
// relative to t0; otherwise from overflow-checked 64-bit ones.  The mode-1 threshold and second bias are
// only formed when mode 1 is chosen.
__device__ __forceinline__ int classify_block(int j0, int64_t tmin, int64_t tmax, const QueryRow& q,
                                              const SeqCtx& sq, ElemCtx& x) {
  const bool full = (j0 + kAttnBN - 1 <= q.r0) && (j0 + kAttnBN <= sq.nh);
  const int pmax_k = position(min(j0 + kAttnBN - 1, sq.L - 1), sq.nh, sq.shared);
  const bool pos_far = q.pmin_q - pmax_k >= sq.R;  // clamped position bias is constant
  // The block's earliest and latest times relative to t0, modulo 2^64 as
  // every time difference of the method is: when both offsets lie within
  // 2^29 of zero (and the wave's rows' do), the difference of any two of the
  // times involved is the difference of their 32-bit offsets, exactly.  The
  // test runs on 32-bit halves, in scalar instructions.
  constexpr uint32_t kNear = 1u << 29;
  const uint64_t emin = (uint64_t)tmin - (uint64_t)sq.t0 + kNear;
  const uint64_t emax = (uint64_t)tmax - (uint64_t)sq.t0 + kNear;
  const bool narrow = q.narrow && (uint32_t)(emin >> 32) == 0u && (uint32_t)emin < 2 * kNear &&
                      (uint32_t)(emax >> 32) == 0u && (uint32_t)emax < 2 * kNear;
  const int32_t dmin = (int32_t)((uint32_t)emin - kNear), dmax = (int32_t)((uint32_t)emax - kNear);
  const int jq = j0 + 4 * (int)((threadIdx.x >> 5) & 1);
  if (full && pos_far && narrow) {
    // The usual far block (wave-uniform test): modes 0 and 1 from 32-bit
    // differences only (|t - t0| < 2^29 for every time involved, so the
    // differences below are exact and span_ok holds); the same values as the
    // general path below, which takes every other case.
    const int32_t lo = q.rq - dmax, hi = q.rq - dmin;
    if (all_lanes((ballot(hi < (1 << 24)) & ballot(lo > -(1 << 24))) | q.idle)) {
      const int bt_lo = time_bucket_med3(lo, sq.bk);
      const int bt_hi = time_bucket_med3(hi, sq.bk);
      x.jq = jq;  // (read only by the inspection dump in these modes)
      if (all_lanes(ballot(bt_hi == bt_lo) | q.idle)) {
        x.c_lo = sq.time_s[bt_lo] + sq.cpos_far;
        return 0;
      }
      if (all_lanes(ballot(bt_hi <= bt_lo + 1) | q.idle)) {
        x.c_lo = sq.time_s[bt_lo] + sq.cpos_far;
        x.c_hi = sq.time_s[bt_hi] + sq.cpos_far;
        x.thr = hi - bucket_floor_small(max(bt_hi, 1), sq.sbits);
        x.rel_off = jq - j0;
        return 1;
      }
    }
  }
  bool novf, span_ok;
  int64_t lo, hi;
  if (narrow) {  // |t - t0| < 2^29 for every time involved: 32-bit differences are exact
    novf = true;
    span_ok = true;
    lo = q.rq - dmax;
    hi = q.rq - dmin;
  } else {
    int64_t span;
    span_ok = !__builtin_sub_overflow(tmax, tmin, &span) && span <= INT32_MAX;
    novf = !__builtin_sub_overflow(q.ts_q, tmax, &lo) && !__builtin_sub_overflow(q.ts_q, tmin, &hi);
  }
  const bool small = novf && hi < (1 << 24) && lo > -(1 << 24);
  const bool all_small = all_lanes(ballot(small) | q.idle);
  int bt_lo, bt_hi;
  if (all_small) {
    bt_lo = time_bucket_med3((int)lo, sq.bk);
    bt_hi = time_bucket_med3((int)hi, sq.bk);
  } else {
    bt_lo = time_bucket(lo, sq.NB, sq.sbits);
    bt_hi = time_bucket(hi, sq.NB, sq.sbits);
  }
  const bool one = novf && bt_lo == bt_hi;
  const bool two = novf && span_ok && bt_hi == bt_lo + 1;
  // Fast modes: no mask, constant position bias, and per row at most two
  // time buckets (decided for the whole wave).
  const bool fast = full && pos_far && all_lanes(ballot(one) | ballot(two) | q.idle);
  const float c_lo = sq.time_s[bt_lo] + sq.cpos_far;
  const bool hist_only = j0 + kAttnBN <= sq.nh;
  const int mode = __builtin_amdgcn_readfirstlane(
      !fast ? (all_small && hist_only ? (full && pos_far ? 4 : 2) : 3) : (all_lanes(ballot(one) | q.idle) ? 0 : 1));
  float c_hi = c_lo;
  int32_t thr = 0;
  if (mode == 1) {
    c_hi = sq.time_s[bt_hi] + sq.cpos_far;
    if (all_small) {
      thr = (int)hi - bucket_floor_small(max(bt_hi, 1), sq.sbits);
    } else {
      const int64_t tt = hi - bucket_floor(max(bt_hi, 1), sq.sbits);
      thr = tt > INT32_MAX ? INT32_MAX : (int32_t)tt;
    }
  }
  x = ElemCtx{jq, q.iq, sq.nh, q.p_q, sq.R, sq.NB, sq.sbits, sq.L, sq.bk, sq.shared, c_lo, c_hi, thr, (int32_t)hi,
              q.p_q - jq, q.iq - jq, sq.pos_s + sq.R + (q.p_q - jq) - 63, sq.cpos_far, q.ts_q, sq.pos_s,
              sq.time_s, jq - j0, sq.ts};
  return mode;
}

// Weights of 32-key half kh in the wave's mode.
__device__ __forceinline__ void half_weights(int mode, const f32x16& sc, float (&p)[16], int kh, const ElemCtx& x,
                                             const int32_t* rb) {
  if (mode == 0)
    elems<0>(sc, p, 32 * kh, x, rb);
  else if (mode == 1)
    elems<1>(sc, p, 32 * kh, x, rb);
  else if (mode == 2)
    elems<2>(sc, p, 32 * kh, x, rb);
  else if (mode == 4)
    elems<4>(sc, p, 32 * kh, x, rb);
  else
    elems<3>(sc, p, 32 * kh, x, rb);
}

// Epilogue of one wave: scale by 1/N_b, per-(row, head) mean and M2 over dv,
// centred AV in the layer dtype and the fp32 statistics.
template <typename T, int DV>
__device__ __forceinline__ void attn_store(f32x16 (&o)[DV / 32], float inv_n, bool qvalid, int64_t row, int h,
                                           int H, void* av, float* stats, int half) {
  float sum = 0.f;
#pragma unroll
  for (int n = 0; n < DV / 32; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o[n][r] *= inv_n;
      sum += o[n][r];
    }
  sum += __shfl_xor(sum, 32, kWave);
  const float mean = sum / (float)DV;
  float m2 = 0.f;
#pragma unroll
  for (int n = 0; n < DV / 32; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float dlt = o[n][r] - mean;
      m2 += dlt * dlt;
    }
  m2 += __shfl_xor(m2, 32, kWave);
  if (!qvalid) return;
  T* dst = reinterpret_cast<T*>(av) + row * (int64_t)(H * DV) + h * DV;
#pragma unroll
  for (int n = 0; n < DV / 32; ++n)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // rows 8g + 4*half + 0..3 of this 32-wide dv tile are consecutive
      T* p = dst + n * 32 + 8 * g + 4 * half;
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = from_f32<T>(o[n][4 * g + e] - mean);
    }
  if (half == 0) {
    stats[(row * H + h) * 2] = mean;
    stats[(row * H + h) * 2 + 1] = m2;
  }
}

// Workgroups per CU the register budget is sized for: three (at most 168
// VGPRs per lane) when a q row plus a k row take at most 256 bytes, else two
// (the token-type step's operands count as 64 bytes more).
constexpr int attn_min_blocks(int row_bytes) { return row_bytes <= 256 ? 3 : 2; }

// CACHED: the queries are candidates only, the keys a cached history of the
// same sequences; every candidate attends the whole history and itself (the
// self term is added in the epilogue), with the shared candidate position.
// TYPED: the bias gains the token-type term table[type_i][type_j], added by
// one more k16 MFMA step per 32-key half: the keys' one-hot types times each
// query row's table row (exact: one-hot entries, table values in the layer
// dtype, fp32 accumulation).
// DUMP (inspection): the same block enumeration, classification and per-pair
// bias selection, but no copies of K and V and no matrix products: each
// selected query row writes the bias of every pair it visits (dump_block).
template <typename T, int DQK, int DV, bool CACHED, bool TYPED, bool DUMP = false>
__global__ __launch_bounds__(256, attn_min_blocks((DQK + DV) * (int)sizeof(T) + (TYPED ? 64 : 0))) void attn_kernel(
    AttnArgs a) {
  typedef AttnCfg<T, DQK, DV> C;
  static_assert(C::NT == 256, "launch bounds assume 4 waves");
  typedef typename Elem<T>::Frag Frag;
  // Two key-block buffers (even / odd blocks), filled asynchronously.
  __shared__ __attribute__((aligned(16))) T Ks0[C::BN * DQK];
  __shared__ __attribute__((aligned(16))) T Ks1[C::BN * DQK];
  __shared__ __attribute__((aligned(16))) T Vs0[C::BN * DV];
  __shared__ __attribute__((aligned(16))) T Vs1[C::BN * DV];
  __shared__ __attribute__((aligned(16))) int32_t rel_s0[C::BN];
  __shared__ __attribute__((aligned(16))) int32_t rel_s1[C::BN];
  __shared__ __attribute__((aligned(16))) int32_t kty_s0[TYPED ? C::BN : 1];
  __shared__ __attribute__((aligned(16))) int32_t kty_s1[TYPED ? C::BN : 1];
  extern __shared__ float tabs[];  // [P] position, [NB] time, [NT * NT] type table of head h
  float* pos_s = tabs + kPosPad;  // entries -kPosPad .. P + kPosPad - 1, the edge values repeated
  float* time_s = tabs + a.P + 2 * kPosPad;
  float* type_s = time_s + a.NB;

  const int H = a.H;
  const int h = blockIdx.x % H;
  const int item = blockIdx.x / H;
  if (item >= a.counts[0]) return;
  const int2 tl = a.tiles[item];
  const SeqInfo si = seq_info(a.off, a.ncand, tl.x, a.T);      // query rows
  const SeqInfo ki = CACHED ? seq_info(a.koff, nullptr, tl.x, a.TK) : si;  // key rows
  const int Lq = si.len;
  const int L = ki.len, nh = CACHED ? ki.len : si.nhist;
  const int64_t s0 = si.start, k0 = ki.start;
  // cached: this item's history chunk (key blocks [clo, chi))
  const int chunk = CACHED ? (tl.y >> 24) : 0;
  int clo = 0, chi = 0;
  if (CACHED) cand_chunk((nh + C::BN - 1) / C::BN, a.nsplit[tl.x], chunk, clo, chi);
  const int i0 = (CACHED ? (tl.y & 0xFFFFFF) : tl.y) * C::BM;
  const int iend = min(i0 + C::BM, Lq);
  const int N_b = CACHED ? L + max(a.mtotal[tl.x], Lq) : L;
  // weights come out scaled by -log2(e) (silu_neglog2e): undone with 1/N_b
  const float inv_n = kNegLn2 / (float)(a.norm_len > 0 ? a.norm_len : N_b);
  const int R = (a.P - 1) / 2;
  const bool shared = a.shared_pos != 0;

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id();
  const int l32 = lane & 31, half = lane >> 5;

  // Key blocks: history [0, min(iend, nh)), then the candidates' own rows; in a
  // cached pass the history chunk's blocks.
  const int a_end = CACHED ? nh : min(iend, nh);
  const int nblk_a = CACHED ? chi - clo : (a_end + C::BN - 1) / C::BN;
  const int b_lo = max(i0, nh), b_hi = iend;
  const int jb0 = max(nblk_a * C::BN, (b_lo / C::BN) * C::BN);
  const int nblk_b = (!CACHED && b_lo < b_hi && jb0 < b_hi) ? (b_hi - jb0 + C::BN - 1) / C::BN : 0;
  const int nblk = nblk_a + nblk_b;
  auto block_start = [&](int blk) __attribute__((always_inline)) {
    return CACHED ? (clo + blk) * C::BN : (blk < nblk_a ? blk * C::BN : jb0 + (blk - nblk_a) * C::BN);
  };

  const T* kg = reinterpret_cast<const T*>(a.k) + ((int64_t)h * a.TK + k0) * DQK;
  const T* vg = reinterpret_cast<const T*>(a.v) + ((int64_t)h * a.TK + k0) * DV;
  TileCopy<T, DQK, C::NW, C::KCPR, true> kcopy;
  TileCopy<T, DV, C::NW, C::VCPR, false> vcopy;
  kcopy.init(w, lane);
  vcopy.init(w, lane);
  // K, V and the keys' time offsets of block `blk` into buffer set (Kb, Vb, rb),
  // and the block's earliest / latest timestamp into tb (read before the
  // copies, so the wait that covers them covers it too).
  auto issue = [&](int blk, T* Kb, T* Vb, int32_t* rb, int32_t* yb, longlong2& tb) __attribute__((always_inline)) {
    const int j0 = block_start(blk);
    // a wave-uniform address, read-only in this kernel: scalar loads
    const __attribute__((address_space(4))) int64_t* t4 =
        reinterpret_cast<const __attribute__((address_space(4))) int64_t*>(
            reinterpret_cast<uintptr_t>(a.tstat + 2 * (k0 + j0)));
    tb.x = t4[0];
    tb.y = t4[1];
    if (!DUMP) {
      kcopy.issue(kg + (int64_t)j0 * DQK, L - j0, Kb, w);
      vcopy.issue(vg + (int64_t)j0 * DV, L - j0, Vb, w);
    }
    // the offsets and types arrays have kAttnBN rows of padding past the key
    // rows, so these never read outside them; entries of rows past the
    // sequence are never used
    if (w == 0)
      __builtin_amdgcn_global_load_lds((glb_void*)(a.rel + k0 + j0 + lane), (lds_void*)rb, 4, 0, 0);
    if (TYPED && w == 1)
      __builtin_amdgcn_global_load_lds((glb_void*)(a.kty + k0 + j0 + lane), (lds_void*)yb, 4, 0, 0);
  };

  // Issue the first block's copies before anything else.
  longlong2 tb0 = {0, 0}, tb1 = {0, 0};
  if (nblk > 0) issue(0, Ks0, Vs0, rel_s0, kty_s0, tb0);

  // Bias tables of head h, as fp32 times -log2(e), into LDS (the weights take
  // s * -log2(e) + bias in one fused multiply-add; the type table stays
  // unscaled: its term is added to the score on the matrix cores).
  for (int i = tid; i < a.P + 2 * kPosPad; i += C::NT)
    tabs[i] = kNegLog2e * to_f32(reinterpret_cast<const T*>(a.pos_tab)[(int64_t)h * a.pos_stride +
                                                                       min(max(i - kPosPad, 0), a.P - 1)]);
  for (int i = tid; i < a.NB; i += C::NT)
    time_s[i] = kNegLog2e * to_f32(reinterpret_cast<const T*>(a.time_tab)[(int64_t)h * a.time_stride + i]);
  if (TYPED)
    for (int i = tid; i < a.NT * a.NT; i += C::NT)
      type_s[i] = to_f32(reinterpret_cast<const T*>(a.type_tab)[(int64_t)h * a.type_stride + i]);

  // This lane's query row and its operand fragments.
  const int r0 = i0 + 32 * w;
  const int rlast = min(r0 + 31, iend - 1);
  const int iq = r0 + l32;
  const bool qvalid = iq < iend;
  const T* qbase = reinterpret_cast<const T*>(a.q) + ((int64_t)h * a.T + s0 + iq) * DQK;
  Frag qf[DQK / 16];
#pragma unroll
  for (int c = 0; c < DQK / 16; ++c) {
    if (qvalid && !DUMP) {
      qf[c] = *reinterpret_cast<const Frag*>(qbase + 16 * c + 8 * half);
    } else {
      qf[c] = Frag{};
    }
  }
  const int64_t ts_q = qvalid ? a.ts[s0 + iq] : 0;
  // A cached pass places every candidate after the whole history at the
  // shared position nh, and masks with row nh - 1 (all history, nothing past it).
  const int p_q = CACHED ? nh : position(iq, nh, shared);
  const int pmin_q = CACHED ? nh : position(r0, nh, shared);
  const bool wave_rows = r0 < iend;

  f32x16 o[DV / 32];
#pragma unroll
  for (int n = 0; n < DV / 32; ++n) o[n] = f32x16{};

  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of block 0 have landed
  __syncthreads();                // ... and every other wave's, plus tables
  const float cpos_far = pos_s[2 * R];  // bias of every pair at distance >= R
  // typed: this lane's query row of the type table, as the B operand of the
  // type step (k = key type 8 * half + e)
  const int ty_q = TYPED && qvalid ? min((int)a.qtypes[s0 + iq], a.NT - 1) : 0;
  Frag wrow{};
  if (TYPED) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 8 * half + e;
      wrow[e] = from_f32<T>(c < a.NT ? type_s[ty_q * a.NT + c] : 0.f);
    }
  }

  // One block of work out of buffer set (Kb, Vb, rb).
  // reference time of the 32-bit classification: the first key row's
  const int64_t t0 = L > 0 ? uniform64(a.kts[k0]) : 0;
  constexpr int64_t kNear = (int64_t)1 << 29;
  int64_t dq = 0;
  const bool q_near = !qvalid || (!__builtin_sub_overflow(ts_q, t0, &dq) && dq > -kNear && dq < kNear);
  const bool q_narrow = __builtin_amdgcn_readfirstlane(__all(q_near) ? 1 : 0) != 0;
  const int32_t rq = qvalid && q_near ? (int32_t)dq : 0;
  const uint64_t idle = ballot(!qvalid);
  const QueryRow qr = CACHED ? QueryRow{nh - 1, nh - 1, nh - 1, p_q, pmin_q, qvalid, ts_q, rq, q_narrow, idle}
                             : QueryRow{r0, rlast, iq, p_q, pmin_q, qvalid, ts_q, rq, q_narrow, idle};
  const SeqCtx sq{L, nh, R, a.NB, a.sbits, small_bucket(a.NB, a.sbits), shared, cpos_far, pos_s, time_s, a.kts + k0, t0};
  float* dump_dst = nullptr;  // inspection: this row's bias row, keys [0, dump_len)
  if (DUMP && qvalid) {
    const int slot = a.dump_slot[s0 + iq];
    if (slot >= 0 && slot < a.dump_slots)
      dump_dst = a.dump + ((int64_t)h * a.dump_slots + slot) * a.dump_len;
  }
  auto consume = [&](int blk, const T* Kb, const T* Vb, const int32_t* rb, const int32_t* yb, int64_t tmin,
                     int64_t tmax) __attribute__((always_inline)) {
    const int j0 = block_start(blk);
    if (!wave_rows || !block_active(j0, qr, sq)) return;
    ElemCtx x;
    const int mode = classify_block(j0, tmin, tmax, qr, sq, x);
    if constexpr (DUMP) {
      if (dump_dst) {
        if (mode == 0)
          dump_block<0>(x, rb, dump_dst, min(L, a.dump_len));
        else if (mode == 1)
          dump_block<1>(x, rb, dump_dst, min(L, a.dump_len));
        else if (mode == 2)
          dump_block<2>(x, rb, dump_dst, min(L, a.dump_len));
        else if (mode == 4)
          dump_block<4>(x, rb, dump_dst, min(L, a.dump_len));
        else
          dump_block<3>(x, rb, dump_dst, min(L, a.dump_len));
      }
      return;
    }
    // Per 32-key half: S^T (K fragments straight from LDS), then this half's
    // V fragments are read while its weights are computed, then P.V.
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x16 sc = f32x16{};
      // Raised wave priority while a wave issues its MFMA chains: the other
      // wave on the SIMD (another workgroup's) then fills the matrix core's
      // busy cycles with its weight arithmetic instead of delaying these
      // issues (measured 1-2% faster).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < DQK / 16; ++c)
        sc = mma_k16(k_frag<T, DQK>(Kb, kh * 32 + l32, 16 * c + 8 * half), qf[c], sc);
      __builtin_amdgcn_s_setprio(0);
      if (TYPED) {
        // one-hot of key kh * 32 + l32's type over k = 8 * half + e (a type
        // outside [0, 16), e.g. in a padding row, gives zeros)
        const int kt = yb[kh * 32 + l32] - 8 * half;
        Frag oh;
#pragma unroll
        for (int e = 0; e < 8; ++e) oh[e] = from_f32<T>(kt == e ? 1.f : 0.f);
        sc = mma_k16(oh, wrow, sc);
      }
      Frag vf[2][DV / 32];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int n = 0; n < DV / 32; ++n) vf[c2][n] = v_frag<T, DV>(Vb, kh * 32 + 16 * c2, n, lane);
      float p[16];
      half_weights(mode, sc, p, kh, x, rb);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const Frag pf = to_frag<T>(p + 8 * c2);
#pragma unroll
        for (int n = 0; n < DV / 32; ++n) o[n] = mma_k16(vf[c2][n], pf, o[n]);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // Block loop, two blocks per trip so each buffer is a distinct LDS object
  // (the compiler then needs no wait on the in-flight copy before reading the
  // other buffer): the copies of block b+1 run while block b is consumed; one
  // barrier per block.
  // The block timestamps move to scalar registers once their load has
  // completed (after the wait that precedes each barrier).
  int64_t tmin0 = uniform64(tb0.x), tmax0 = uniform64(tb0.y), tmin1 = 0, tmax1 = 0;
  for (int blk = 0; blk < nblk; blk += 2) {
    if (blk + 1 < nblk) issue(blk + 1, Ks1, Vs1, rel_s1, kty_s1, tb1);
    consume(blk, Ks0, Vs0, rel_s0, kty_s0, tmin0, tmax0);
    if (blk + 1 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    tmin1 = uniform64(tb1.x);
    tmax1 = uniform64(tb1.y);
    if (blk + 2 < nblk) issue(blk + 2, Ks0, Vs0, rel_s0, kty_s0, tb0);
    consume(blk + 1, Ks1, Vs1, rel_s1, kty_s1, tmin1, tmax1);
    if (blk + 2 >= nblk) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    tmin0 = uniform64(tb0.x);
    tmax0 = uniform64(tb0.y);
  }

  if (DUMP || r0 >= iend) return;
  if (CACHED && qvalid && chunk == 0) {
    // The candidate's own key: distance 0 (bucket R), time difference 0
    // (bucket 0).  q.k over this lane's half of dqk, then across the halves.
    const T* ks = reinterpret_cast<const T*>(a.qk) + ((int64_t)h * a.T + s0 + iq) * DQK;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < DQK / 16; ++c) {
      const Frag kf = *reinterpret_cast<const Frag*>(ks + 16 * c + 8 * half);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += to_f32(qf[c][e]) * to_f32(kf[e]);
    }
    dot += __shfl_xor(dot, 32, kWave);
    const float wself = silu_neglog2e(dot + (TYPED ? type_s[ty_q * a.NT + ty_q] : 0.f), pos_s[R] + time_s[0]);
    const T* vs = reinterpret_cast<const T*>(a.qv) + ((int64_t)h * a.T + s0 + iq) * DV;
#pragma unroll
    for (int n = 0; n < DV / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[n][r] += wself * to_f32(vs[32 * n + 8 * (r >> 2) + 4 * half + (r & 3)]);
  }
  if (CACHED) {
    // this chunk's share, scaled; cand_gate_kernel sums the chunks
    if (!qvalid) return;
    float* dst = a.part + ((int64_t)chunk * a.T + s0 + iq) * (H * DV) + h * DV;
#pragma unroll
    for (int n = 0; n < DV / 32; ++n)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(dst + n * 32 + 8 * g + 4 * half) =
            make_float4(o[n][4 * g] * inv_n, o[n][4 * g + 1] * inv_n, o[n][4 * g + 2] * inv_n,
                        o[n][4 * g + 3] * inv_n);
    return;
  }
  attn_store<T, DV>(o, inv_n, qvalid, s0 + iq, h, H, a.av, a.stats, half);
}

template <typename T, int DQK, int DV>
static hipError_t launch_t(const AttnArgs& a, bool cached, int64_t grid, hipStream_t s) {
  const bool typed = a.NT > 0;
  const size_t shmem = (size_t)(a.P + 2 * kPosPad + a.NB + (typed ? a.NT * a.NT : 0)) * sizeof(float);
  const dim3 g((unsigned)grid), b(AttnCfg<T, DQK, DV>::NT);
  if (cached && typed)
    hipLaunchKernelGGL((attn_kernel<T, DQK, DV, true, true>), g, b, shmem, s, a);
  else if (cached)
    hipLaunchKernelGGL((attn_kernel<T, DQK, DV, true, false>), g, b, shmem, s, a);
  else if (typed)
    hipLaunchKernelGGL((attn_kernel<T, DQK, DV, false, true>), g, b, shmem, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, DQK, DV, false, false>), g, b, shmem, s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dims(const AttnArgs& a, bool cached, int dqk, int dv, int64_t grid, hipStream_t s) {
#define HSTU_ATTN_CASE(Q, V_) \
  if (dqk == Q && dv == V_) return launch_t<T, Q, V_>(a, cached, grid, s);
  HSTU_ATTN_CASE(32, 32)
  HSTU_ATTN_CASE(32, 64)
  HSTU_ATTN_CASE(32, 128)
  HSTU_ATTN_CASE(64, 32)
  HSTU_ATTN_CASE(64, 64)
  HSTU_ATTN_CASE(64, 128)
  HSTU_ATTN_CASE(128, 32)
  HSTU_ATTN_CASE(128, 64)
  HSTU_ATTN_CASE(128, 128)
#undef HSTU_ATTN_CASE
  return hipErrorInvalidValue;
}

// fp32 layers: head widths up to 64 (the API rejects wider ones for fp32).
static hipError_t launch_dims_f32(const AttnArgs& a, bool cached, int dqk, int dv, int64_t grid, hipStream_t s) {
  if (dqk == 32 && dv == 32) return launch_t<float, 32, 32>(a, cached, grid, s);
  if (dqk == 32 && dv == 64) return launch_t<float, 32, 64>(a, cached, grid, s);
  if (dqk == 64 && dv == 32) return launch_t<float, 64, 32>(a, cached, grid, s);
  if (dqk == 64 && dv == 64) return launch_t<float, 64, 64>(a, cached, grid, s);
  return hipErrorInvalidValue;
}

static AttnArgs attn_args(const hstu_desc& d, const AttnRows& r, const hstu_bias_tables& tab, const void* q,
                          const void* k, const void* v, const void* qk, const void* qv, float* part, void* av,
                          float* stats, const AttnScratch& sc) {
  AttnArgs a{};
  a.part = part;
  a.nsplit = sc.nsplit;
  a.NT = r.types.nt;
  a.qtypes = r.types.q;
  a.kty = sc.kty;
  a.type_tab = tab.type;
  a.type_stride = tab.type_head_stride;
  a.off = r.qoff;
  a.ncand = r.ncand;
  a.ts = r.qts;
  a.koff = r.koff;
  a.kts = r.kts;
  a.mtotal = r.mtotal;
  a.pos_tab = tab.pos;
  a.time_tab = tab.time;
  a.q = q;
  a.k = k;
  a.v = v;
  a.qk = qk;
  a.qv = qv;
  a.av = av;
  a.stats = stats;
  a.tiles = sc.tiles;
  a.counts = sc.counts;
  a.rel = sc.rel;
  a.tstat = sc.tstat;
  a.T = r.Tq;
  a.TK = r.Tk;
  a.H = d.num_heads;
  a.P = d.pos_buckets;
  a.NB = d.time_buckets;
  a.sbits = d.time_sub_bits;
  a.pos_stride = tab.pos_head_stride;
  a.time_stride = tab.time_head_stride;
  a.norm_len = d.norm_len;
  a.shared_pos = (d.flags & HSTU_CAND_SHARED_POS) ? 1 : 0;
  return a;
}

static hipError_t launch_attn_impl(const hstu_desc& d, const AttnRows& r, const hstu_bias_tables& tab,
                                   const void* q, const void* k, const void* v, const void* qk, const void* qv,
                                   float* part, void* av, float* stats, const AttnScratch& sc, hipStream_t s) {
  if (r.Tq == 0) return hipSuccess;
  const AttnArgs a = attn_args(d, r, tab, q, k, v, qk, qv, part, av, stats, sc);
  const int64_t grid = attn_max_items(r.Tq, r.B, r.cached) * d.num_heads;
  if (d.dtype == HSTU_BF16) return launch_dims<bf16>(a, r.cached, d.dqk, d.dv, grid, s);
  return launch_dims_f32(a, r.cached, d.dqk, d.dv, grid, s);
}

hipError_t launch_attn(const hstu_desc& d, const AttnRows& r, const hstu_bias_tables& tab, const void* q,
                       const void* k, const void* v, const void* qk, const void* qv, void* av, float* stats,
                       const AttnScratch& sc, hipStream_t s) {
  if (r.cached) return hipErrorInvalidValue;  // needs the partial buffer: launch_attn_cached
  return launch_attn_impl(d, r, tab, q, k, v, qk, qv, nullptr, av, stats, sc, s);
}

hipError_t launch_attn_dump(const hstu_desc& d, const AttnRows& r, const hstu_bias_tables& tab,
                            const int32_t* slot, int nslots, int len, float* out, const AttnScratch& sc,
                            hipStream_t s) {
  if (r.cached || r.types.nt > 0) return hipErrorInvalidValue;
  if (r.Tq == 0 || nslots == 0 || len == 0) return hipSuccess;
  AttnArgs a = attn_args(d, r, tab, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, sc);
  a.dump = out;
  a.dump_slot = slot;
  a.dump_slots = nslots;
  a.dump_len = len;
  const size_t shmem = (size_t)(a.P + 2 * kPosPad + a.NB) * sizeof(float);
  const dim3 g((unsigned)(attn_max_items(r.Tq, r.B, false) * d.num_heads)), b(kAttnBM / 32 * kWave);
  if (d.dtype == HSTU_BF16)
    hipLaunchKernelGGL((attn_kernel<bf16, 32, 32, false, false, true>), g, b, shmem, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<float, 32, 32, false, false, true>), g, b, shmem, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_cached(const hstu_desc& d, const AttnRows& r, const hstu_bias_tables& tab,
                              const void* q, const void* k, const void* v, const void* qk, const void* qv,
                              float* part, const AttnScratch& sc, hipStream_t s) {
  if (!r.cached) return hipErrorInvalidValue;
  return launch_attn_impl(d, r, tab, q, k, v, qk, qv, part, nullptr, nullptr, sc, s);
}

}  // namespace hstu
