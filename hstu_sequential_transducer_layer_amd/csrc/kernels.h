// Host-side launchers of the HSTU kernels (one translation unit per stage).
// All take device pointers, enqueue on `stream` and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu.h"

namespace hstu {

// Query-row tile of the attention kernel and key block it streams.
constexpr int kAttnBM = 128;
constexpr int kAttnBN = 64;

// A cached candidate pass splits each sequence's history into
// min(kCandMaxSplit, ceil(key blocks / kCandSplitBlocks)) chunks (at least one),
// each its own work item, so that a micro-batch with few query tiles still
// fills the chip.  The split depends only on the history length, so a row's
// result does not depend on the micro-batch it is scored in.
constexpr int kCandSplitBlocks = 4;
constexpr int kCandMaxSplit = 8;

__host__ __device__ inline int cand_nsplit(int hist_len) {
  const int nb = (hist_len + kAttnBN - 1) / kAttnBN;
  const int s = (nb + kCandSplitBlocks - 1) / kCandSplitBlocks;
  return s < 1 ? 1 : (s > kCandMaxSplit ? kCandMaxSplit : s);
}
// Key blocks [lo, hi) of history chunk c out of ns over nblk blocks (balanced;
// empty only when nblk = 0).
__host__ __device__ inline void cand_chunk(int nblk, int ns, int c, int& lo, int& hi) {
  lo = c * nblk / ns;
  hi = (c + 1) * nblk / ns;
}

// Upper bound on attention work items (q-tiles over all sequences).
inline int64_t attn_max_tiles(int64_t T, int32_t B) { return (T + kAttnBM - 1) / kAttnBM + B; }
inline int64_t attn_max_items(int64_t Tq, int32_t B, bool cached) {
  return attn_max_tiles(Tq, B) * (cached ? kCandMaxSplit : 1);
}
// Upper bound on key blocks (64 keys from a sequence's start) over all sequences.
inline int64_t attn_max_kblocks(int64_t T, int32_t B) { return (T + kAttnBN - 1) / kAttnBN + B; }

// Device scratch of the attention stage, carved from one caller buffer.  Tq
// counts query rows, Tk key rows (the same rows in a layer pass; the cached
// history in a candidate pass).
//   tiles   int2 {b, q-tile}, work list ordered by decreasing cost; in a
//           cached pass {b, q-tile | history chunk << 24}
//   kblocks int2 {b, key block}, every key block once, any order
//   counts  int32 [2]: number of tiles, number of key blocks
//   tbase, kbase  int32 [B + 1]: first tile / key block of each sequence
//   nsplit  int32 [B]: history chunks per sequence (cached pass; else 1)
//   rel     int32 [Tk + kAttnBN]: ts[row] - (earliest timestamp of its key block)
//   tstat   int64 [Tk][2]: at each key block's first row, the block's
//           earliest and latest timestamps (other rows unused)
//   kty     int32 [Tk + kAttnBN]: key rows' token types (typed layers)
struct AttnScratch {
  int2* tiles;
  int2* kblocks;
  int32_t* counts;
  int32_t* tbase;
  int32_t* kbase;
  int32_t* nsplit;
  int32_t* rel;
  int64_t* tstat;
  int32_t* kty;
};

inline size_t attn_align(size_t n) { return (n + 255) & ~(size_t)255; }

inline size_t attn_scratch_bytes(int64_t Tq, int64_t Tk, int32_t B, bool cached) {
  return attn_align((size_t)attn_max_items(Tq, B, cached) * 8) + attn_align((size_t)attn_max_kblocks(Tk, B) * 8) +
         attn_align(2 * sizeof(int32_t)) + 3 * attn_align(((size_t)B + 1) * 4) +
         2 * attn_align((size_t)(Tk + kAttnBN) * 4) + attn_align((size_t)Tk * 16);
}
inline size_t attn_scratch_bytes(int64_t T, int32_t B) { return attn_scratch_bytes(T, T, B, false); }

inline AttnScratch attn_scratch(void* base, int64_t Tq, int64_t Tk, int32_t B, bool cached) {
  char* p = (char*)base;
  AttnScratch a;
  a.tiles = (int2*)p;
  p += attn_align((size_t)attn_max_items(Tq, B, cached) * 8);
  a.kblocks = (int2*)p;
  p += attn_align((size_t)attn_max_kblocks(Tk, B) * 8);
  a.counts = (int32_t*)p;
  p += attn_align(2 * sizeof(int32_t));
  a.tbase = (int32_t*)p;
  p += attn_align(((size_t)B + 1) * 4);
  a.kbase = (int32_t*)p;
  p += attn_align(((size_t)B + 1) * 4);
  a.nsplit = (int32_t*)p;
  p += attn_align(((size_t)B + 1) * 4);
  a.rel = (int32_t*)p;
  p += attn_align((size_t)(Tk + kAttnBN) * 4);
  a.tstat = (int64_t*)p;
  p += attn_align((size_t)Tk * 16);
  a.kty = (int32_t*)p;
  return a;
}
inline AttnScratch attn_scratch(void* base, int64_t T, int32_t B) { return attn_scratch(base, T, T, B, false); }

// Partial AV of a cached pass: [kCandMaxSplit][Tq][H * dv] fp32, chunk c of
// row r at (c * Tq + r) * H * dv (only each sequence's nsplit chunks written).
inline size_t cand_partial_bytes(int64_t Tq, int H, int dv) {
  return attn_align((size_t)kCandMaxSplit * (size_t)Tq * (size_t)H * (size_t)dv * 4);
}

// Token types of a pass (num_types > 0): the query rows' and the key rows'.
struct AttnTypes {
  const uint8_t* q;
  const uint8_t* k;
  int nt;  // 0: no type term
};

// The rows an attention pass reads.  Query rows: sequence b is
// [qoff[b], qoff[b + 1]) of the query-side tensors, its last ncand[b] rows
// candidates.  Key rows: in a layer pass the same rows (koff = qoff, kts = the
// query timestamps); in a cached candidate pass the queries are candidates
// only and the keys are the history [koff[b], koff[b + 1]) of the cache,
// mtotal[b] being the sequence's full candidate count (for N_b).
struct AttnRows {
  const int64_t* qoff;
  const int32_t* ncand;
  const int64_t* qts;
  int64_t Tq;
  const int64_t* koff;
  const int64_t* kts;
  int64_t Tk;
  const int32_t* mtotal;  // cached pass only
  int32_t B;
  bool cached;
  AttnTypes types;
};

// --- prep.hip
hipError_t launch_ln_in(hstu_dtype dt, const void* x, const void* g, const void* b, void* y,
                        int64_t T, int d, float eps, hipStream_t s);
// Attention preparation: the work list (one workgroup), then the per-key-block
// time-stamp summary (tstat, rel) that the attention kernel reads per block.
hipError_t launch_attn_prep(const AttnRows& rows, int bm, const AttnScratch& sc, hipStream_t s);

// --- proj.hip: u|v|q|k = SiLU(xn W1^T + b1), scattered to the stage layouts;
// when pre is not null also the pre-activation xn W1^T + b1 itself, [T, N1]
// row-major in the layer dtype (the backward's SiLU derivative reads it).
hipError_t launch_proj(const hstu_desc& d, const void* xn, int64_t T, const void* w1,
                       const void* b1, void* u, void* v, void* q, void* k, void* pre, hipStream_t s);

// --- attn.hip: av, stats of the query rows.  k, v: the key rows' tensors (in
// a cached pass the history cache; q, qk, qv are then the candidates' own
// tensors, qk / qv giving each candidate's self term).
hipError_t launch_attn(const hstu_desc& d, const AttnRows& rows, const hstu_bias_tables& tab, const void* q,
                       const void* k, const void* v, const void* qk, const void* qv, void* av, float* stats,
                       const AttnScratch& sc, hipStream_t s);
// Cached pass: the attention writes each history chunk's partial AV (scaled
// by 1/N_b; the candidate's own term in chunk 0) to `part`.
hipError_t launch_attn_cached(const hstu_desc& d, const AttnRows& rows, const hstu_bias_tables& tab,
                              const void* q, const void* k, const void* v, const void* qk, const void* qv,
                              float* part, const AttnScratch& sc, hipStream_t s);
// Inspection: the attention kernel's per-pair biases (times -log2 e) for the
// query rows with slot[row] in [0, nslots): out[h][slot][j], j < len.
hipError_t launch_attn_dump(const hstu_desc& d, const AttnRows& rows, const hstu_bias_tables& tab,
                            const int32_t* slot, int nslots, int len, float* out, const AttnScratch& sc,
                            hipStream_t s);

// --- out.hip: z = LN_av(av) * u, then out = z W2^T + b2 (+ x).
hipError_t launch_gate(const hstu_desc& d, int64_t T, const hstu_weights& w, const void* u,
                       const void* av, const float* stats, void* z, hipStream_t s);
hipError_t launch_f2(const hstu_desc& d, const void* x, int64_t T, const hstu_weights& w,
                     const void* z, void* out, hipStream_t s);
// Cached pass: z = (LayerNorm(sum of the row's history chunks) * g + b) * u,
// the chunks summed in chunk order (query rows qoff / B / Tq of the pass).
hipError_t launch_cand_gate(const hstu_desc& d, const int64_t* qoff, int32_t B, int64_t Tq,
                            const int32_t* nsplit, const float* part, const hstu_weights& w, const void* u,
                            void* z, hipStream_t s);

// --- sl.hip: stochastic length (plan + selection) and the row gather.
hipError_t launch_sl_sample(const int64_t* off, int32_t B, int64_t T, const float* u, const uint32_t* keys,
                            double thr, int64_t k, double na, int64_t* new_off, int64_t* rows, int32_t* trunc,
                            hipStream_t s);
hipError_t launch_gather_rows(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* rows,
                              const int64_t* count, int64_t max_rows, void* dst, hipStream_t s);

// --- attn_bwd.hip: dq, dv, dk into dact (fp32 [T, N1], columns of the
// u|v|q|k split) and the bias-table gradients (tab_part: [max items * H][P + NB]).
// With pre (the forward's saved pre-activation [T, N1], layer dtype) the
// gradients go out times SiLU'(pre) into dpre (same layout and dtype) instead
// of into dact.
hipError_t launch_attn_bwd(const hstu_desc& d, const int64_t* off, const int32_t* ncand, int32_t B, int64_t T,
                           const int64_t* ts, const hstu_bias_tables& tab, const void* q, const void* k,
                           const void* v, const void* dout, float* dact, const void* pre, void* dpre,
                           float* tab_part, float* gpos, float* gtime, const AttnScratch& sc, hipStream_t s);
// C [M, N] = A^T B (fp32) over K rows of the row-major bf16 A [K, M] and
// B [K, N] (M, N multiples of 8): weight gradients over the token dimension
// without transposed copies; split over K into split_buf (split_cap floats)
// when the tiles alone would leave compute units idle.
hipError_t launch_gemm_tn_f32(const void* A, const void* B, float* C, int M, int N, int64_t K, float* split_buf,
                              int64_t split_cap, hipStream_t s);

// --- bwd.hip
size_t colsum_tmp_bytes(int64_t R, int64_t C);
hipError_t launch_colsum(hstu_dtype dt_in, bool in_f32, const void* src, int64_t R, int64_t C, float* tmp,
                         float* dst, hipStream_t s);
hipError_t launch_transpose(hstu_dtype dt, const void* src, int64_t R, int64_t C, int64_t Rp, void* dst,
                            hipStream_t s);
// C [M, N] fp32 = A [M, K] B [N, K]^T (K a multiple of 8).  With split_buf
// (kGemmMaxSplit * M * N floats) a long K is split over up to kGemmMaxSplit
// workgroups per tile when the tiles alone would not fill the chip.
constexpr int kGemmMaxSplit = 8;
hipError_t launch_gemm_nt_f32(hstu_dtype dt, const void* A, const void* Bm, float* C, int64_t M, int N, int K,
                              float* split_buf, hipStream_t s);
// gpart, bpart: ceil(T / 32) x H*dv partial rows of the LayerNorm_av gain and
// offset gradients, summed into dg, db.
// dU goes out as its pre-activation gradient dU * SiLU'(pre) into the u
// columns of dpre [T, N1] (layer dtype), pre the forward's saved
// pre-activation.
hipError_t launch_gate_bwd(const hstu_desc& d, int64_t T, const hstu_weights& w, const float* dz, const void* u,
                           const void* av, const float* stats, const void* pre, void* dpre, void* dav, float* gpart,
                           float* bpart, float* dg, float* db, hipStream_t s);
// gpart, bpart: ceil(T / 32) x d_model partial rows of the LayerNorm_in gain
// and offset gradients, summed into dg, db (zero without HSTU_INPUT_NORM).
hipError_t launch_ln_bwd(const hstu_desc& d, const void* x, const float* dxn, const hstu_weights& w, const void* dy,
                         int64_t T, void* dx, float* gpart, float* bpart, float* dg, float* db, hipStream_t s);

// --- debug.hip
hipError_t launch_debug_indices(const hstu_desc& d, const int64_t* off, const int32_t* ncand,
                                int32_t B, int64_t T, const int64_t* ts, const int64_t* pairs,
                                int64_t n, int64_t* out, hipStream_t s);

}  // namespace hstu
