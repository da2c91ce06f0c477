// Device-side building blocks shared by the HSTU kernels (gfx950 / CDNA4).
//
// MFMA convention used everywhere: one "k16 step" of a 32x32 output tile.
//   A operand  lane l holds row (l % 32) and the eight k-values 8*(l/32) .. +7
//   B operand  lane l holds column (l % 32) and the same eight k-values
//   C (f32x16) lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4)
// For bf16 that is one v_mfma_f32_32x32x16_bf16.  For fp32 it is eight
// v_mfma_f32_32x32x2_f32, the e-th contracting k-value e of each lane half; the
// output layout is identical, so every kernel is written once for both types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Index of the calling wave within its workgroup, as a wave-uniform (scalar)
// value: the compiler cannot infer that threadIdx.x / 64 is uniform, and
// branches on values derived from it would otherwise be compiled as divergent
// (every wave issuing every side under an exec mask).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A wave-uniform 64-bit value moved to scalar registers (both halves).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <typename T>
struct Elem;
template <>
struct Elem<bf16> {
  typedef bf16x8 Frag;                 // one k16 step of an MFMA operand
  static constexpr int kVec = 8;       // elements per 16-byte vector
};
template <>
struct Elem<float> {
  typedef f32x8 Frag;
  static constexpr int kVec = 4;
};

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }

__device__ __forceinline__ f32x16 mma_k16(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_k16(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

// 16-byte vector load/store of kVec elements.
template <typename T>
__device__ __forceinline__ uint4 ld16(const T* p) { return *reinterpret_cast<const uint4*>(p); }
template <typename T>
__device__ __forceinline__ void st16(T* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ void unpack(const uint4& v, float (&o)[8], bf16) {
  const bf16* e = reinterpret_cast<const bf16*>(&v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)e[i];
}
__device__ __forceinline__ void unpack(const uint4& v, float (&o)[4], float) {
  const float* e = reinterpret_cast<const float*>(&v);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = e[i];
}
__device__ __forceinline__ uint4 pack(const float (&o)[8], bf16) {
  uint4 v;
  bf16* e = reinterpret_cast<bf16*>(&v);
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (bf16)o[i];
  return v;
}
__device__ __forceinline__ uint4 pack(const float (&o)[4], float) {
  uint4 v;
  float* e = reinterpret_cast<float*>(&v);
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = o[i];
  return v;
}

// SiLU(z) = z * sigmoid(z) = z / (1 + 2^(-z*log2(e))).  For z < -88 the power
// overflows to +inf and the quotient is -0, the correct limit; no NaN arises.
__device__ __forceinline__ float silu(float z) {
  float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// SiLU'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))).
__device__ __forceinline__ float silu_grad(float z) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
  return sg * (1.0f + z * (1.0f - sg));
}

// -log2(e) * SiLU(s + b), given bn = -log2(e) * b: z' = -log2(e) (s + b) in one
// fused multiply-add, then z' / (1 + 2^z').  Callers fold the constant
// -ln(2) = 1 / -log2(e) into a later scale.
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;
__device__ __forceinline__ float silu_neglog2e(float s, float bn) {
  const float z = __builtin_fmaf(s, kNegLog2e, bn);
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// Lane masks of the wave in scalar registers.  A comparison's ballot is the
// mask the comparison itself writes, so testing "every lane that counts"
// as ballot(cmp) | (mask of lanes that do not count) == exec costs no
// vector instruction beyond the comparison.
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ bool all_lanes(uint64_t m) { return m == __builtin_amdgcn_read_exec(); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---------------------------------------------------------------- indexing
// Jagged metadata, clamped so that malformed offsets or candidate counts can
// never address rows outside [0, T).
struct SeqInfo {
  int64_t start;  // first flat row
  int32_t len;    // L_b
  int32_t nhist;  // n_b = L_b - m_b
};

__device__ __forceinline__ SeqInfo seq_info(const int64_t* off, const int32_t* ncand, int b,
                                            int64_t T) {
  int64_t s0 = off[b], s1 = off[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > T ? T : s0);
  s1 = s1 < s0 ? s0 : (s1 > T ? T : s1);
  SeqInfo si;
  si.start = s0;
  si.len = (int32_t)(s1 - s0);
  int32_t m = ncand ? ncand[b] : 0;
  m = m < 0 ? 0 : (m > si.len ? si.len : m);
  si.nhist = si.len - m;
  return si;
}

// Log-bucketed time difference: 0 for dt <= 0, else 1 + (k << s) + the s bits
// right below the leading one of dt, k = floor(log2 dt), capped at nb - 1.
// Written with selects only (no per-lane branch), so that callers inside
// wave-uniform branches keep those branches.
__device__ __forceinline__ int time_bucket(int64_t dt, int nb, int s) {
  const int k = 63 - __clzll((unsigned long long)(dt | 1));
  const int64_t below = (k >= s) ? (dt >> (k - s)) : (dt << (s - k));
  int b = 1 + (k << s) + (int)(below & ((1 << s) - 1));
  b = b < nb - 1 ? b : nb - 1;
  return dt > 0 ? b : 0;
}

// Log time bucket of dt for |dt| < 2^24, where (float)dt is exact: its bits
// hold the exponent floor(log2 dt) + 127 followed by the mantissa, so
// bits >> (23 - s) = ((k + 127) << s) | (the s bits below the leading one).
// dt <= 0 gives a value below 1 (the bits of a negative float are negative as
// int32), which the clamp sends to bucket 0.  Equal to time_bucket there.
__device__ __forceinline__ int time_bucket_small(int dt, int nb, int s) {
  const int b = (__float_as_int((float)dt) >> (23 - s)) + 1 - (127 << s);
  return min(max(b, 0), nb - 1);
}

// The same bucket with the clamp done by one float median instead of an
// integer max and min: lo and hi are the smallest floats whose bits give
// bucket 0 and bucket nb - 1 (hi capped at 2^24, above every dt of this
// path), so clamping float(dt) to [lo, hi] clamps the bucket to [0, nb - 1].
// tests/test_bucket_clamp_host.py restates the formula and checks it against
// the oracle's bucket for every sub-bucket count the library accepts.
struct SmallBucket {
  float lo, hi;
  int sh, add;
};
__device__ __forceinline__ SmallBucket small_bucket(int nb, int s) {
  const int top = (nb - 2 + (127 << s)) << (23 - s);  // bits of the first float of bucket nb - 1
  return SmallBucket{__int_as_float(((127 << s) - 1) << (23 - s)),
                     __int_as_float(min(top, __float_as_int(16777216.0f))), 23 - s, 1 - (127 << s)};
}
__device__ __forceinline__ int time_bucket_med3(int dt, const SmallBucket& k) {
  return (__float_as_int(__builtin_amdgcn_fmed3f((float)dt, k.lo, k.hi)) >> k.sh) + k.add;
}

// Smallest dt >= 1 whose time bucket is >= b, for a bucket b >= 1 that some
// dt in int64 reaches.  With c = b - 1 = (k << s) + sub: for k >= s every
// sub-bucket exists and starts at 2^k + sub * 2^(k-s); for k < s the bits
// below dt's leading one are zero-extended, so only sub-buckets whose low
// s - k bits are zero exist and the answer rounds sub up to the next one.
__device__ __forceinline__ int64_t bucket_floor(int b, int s) {
  const int c = b - 1, k = c >> s, sub = c & ((1 << s) - 1);
  if (k >= s) return ((int64_t)1 << k) | ((int64_t)sub << (k - s));
  const int sh = s - k;
  return ((int64_t)1 << k) + (((int64_t)sub + (1 << sh) - 1) >> sh);
}

__device__ __forceinline__ int64_t wrap_sub(int64_t a, int64_t b) {
  return (int64_t)((uint64_t)a - (uint64_t)b);
}

__device__ __forceinline__ int pos_bucket(int pi, int pj, int R) { return min(max(pi - pj, -R), R) + R; }

__device__ __forceinline__ int position(int i, int nhist, bool shared) {
  return shared ? (i < nhist ? i : nhist) : i;
}

__device__ __forceinline__ bool attends(int i, int j, int nhist) {
  return j <= i && (j < nhist || j == i);
}

}  // namespace hstu
