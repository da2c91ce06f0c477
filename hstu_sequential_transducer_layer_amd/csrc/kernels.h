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

// Upper bound on attention work items (q-tiles over all sequences).
inline int64_t attn_max_tiles(int64_t T, int32_t B) { return (T + kAttnBM - 1) / kAttnBM + B; }

// --- prep.hip
hipError_t launch_ln_in(hstu_dtype dt, const void* x, const void* g, const void* b, void* y,
                        int64_t T, int d, float eps, hipStream_t s);
// Builds the attention work list: int2 {b, q-tile} ordered by decreasing cost,
// count stored at tiles_count.  One workgroup.
hipError_t launch_build_tiles(const int64_t* off, const int32_t* ncand, int32_t B, int64_t T,
                              int2* tiles, int32_t* tiles_count, hipStream_t s);

// --- proj.hip: u|v|q|k = SiLU(xn W1^T + b1), scattered to the stage layouts.
hipError_t launch_proj(const hstu_desc& d, const void* xn, int64_t T, const void* w1,
                       const void* b1, void* u, void* v, void* q, void* k, hipStream_t s);

// --- attn.hip
hipError_t launch_attn(const hstu_desc& d, const int64_t* off, const int32_t* ncand, int32_t B,
                       int64_t T, const int64_t* ts, const hstu_bias_tables& tab, const void* q,
                       const void* k, const void* v, void* av, float* stats, const int2* tiles,
                       const int32_t* tiles_count, hipStream_t s);

// --- out.hip: z = LN_av(av) * u, then out = z W2^T + b2 (+ x).
hipError_t launch_gate(const hstu_desc& d, int64_t T, const hstu_weights& w, const void* u,
                       const void* av, const float* stats, void* z, hipStream_t s);
hipError_t launch_f2(const hstu_desc& d, const void* x, int64_t T, const hstu_weights& w,
                     const void* z, void* out, hipStream_t s);

// --- debug.hip
hipError_t launch_debug_indices(const hstu_desc& d, const int64_t* off, const int32_t* ncand,
                                int32_t B, int64_t T, const int64_t* ts, const int64_t* pairs,
                                int64_t n, int64_t* out, hipStream_t s);

}  // namespace hstu
