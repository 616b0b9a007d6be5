// Device helpers for the gfx950 (CDNA4) verification kernels: bf16 unpacking and
// 64-lane wavefront reductions built from DPP row permutes and the gfx950
// permlane16/32 swaps.
//
// Every reduction here has a fixed combination tree, so results are bitwise
// reproducible run to run (no atomics on floating-point data anywhere).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
// fp32 log2(e); the kernels evaluate exp(x) as exp2(x * kL2E).  The same fp32
// constant is used everywhere a normaliser is formed or consumed, so the whole
// path computes softmax(kL2E * ln(2) * l), a temperature within 1.3e-8 of 1.
constexpr float kL2E = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight consecutive bf16 values (one 16-byte load) widened to fp32.
__device__ __forceinline__ void unpack8(const uint4& w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// ---------------------------------------------------------------- fp64 exp2 / log2
// Inlined double-precision 2^x and log2(x) for the per-row finalize (the library versions
// are large enough to be emitted as calls, which costs the streaming kernels registers).
// exp2_d: 2^x = 2^n e^(f ln2), n = floor(x), f in [0, 1); Taylor series of e^t to t^13
// (|t| < 0.7: truncation below 2^-53 relative).  log2_d: x = m 2^e, m in [0.5, 1); the fp32
// hardware log2 of m refined by one Newton step on 2^y = m (error squared: ~1e-15).
__device__ __forceinline__ double exp2_d(double x) {
  if (!(x > -1100.0)) return 0.0;
  if (x > 1100.0) return __builtin_inf();
  const double n = floor(x);
  const double t = (x - n) * 0.69314718055994530942;
  double p = 1.0 / 6227020800.0;  // 1/13!
  p = fma(p, t, 1.0 / 479001600.0);
  p = fma(p, t, 1.0 / 39916800.0);
  p = fma(p, t, 1.0 / 3628800.0);
  p = fma(p, t, 1.0 / 362880.0);
  p = fma(p, t, 1.0 / 40320.0);
  p = fma(p, t, 1.0 / 5040.0);
  p = fma(p, t, 1.0 / 720.0);
  p = fma(p, t, 1.0 / 120.0);
  p = fma(p, t, 1.0 / 24.0);
  p = fma(p, t, 1.0 / 6.0);
  p = fma(p, t, 0.5);
  p = fma(p, t, 1.0);
  p = fma(p, t, 1.0);
  return ldexp(p, static_cast<int>(n));
}

// exp2_bulk: exp2_d for sums over many columns, with no branch, so that the compiler can
// interleave the independent evaluations of a lane's columns (one evaluation alone is a chain
// of dependent fp64 operations).  x is clamped to [-1100, 1100] (2^-1100 rounds to 0, as
// exp2_d's -inf and underflow); the reduction is to the nearest integer, f in [-1/2, 1/2],
// |t| < 0.35, so the Taylor series to t^12 is exact to below 2^-53 relative.
__device__ __forceinline__ double exp2_bulk(double x) {
  x = fmin(fmax(x, -1100.0), 1100.0);
  const double n = rint(x);
  const double t = (x - n) * 0.69314718055994530942;
  double p = 1.0 / 479001600.0;  // 1/12!
  p = fma(p, t, 1.0 / 39916800.0);
  p = fma(p, t, 1.0 / 3628800.0);
  p = fma(p, t, 1.0 / 362880.0);
  p = fma(p, t, 1.0 / 40320.0);
  p = fma(p, t, 1.0 / 5040.0);
  p = fma(p, t, 1.0 / 720.0);
  p = fma(p, t, 1.0 / 120.0);
  p = fma(p, t, 1.0 / 24.0);
  p = fma(p, t, 1.0 / 6.0);
  p = fma(p, t, 0.5);
  p = fma(p, t, 1.0);
  p = fma(p, t, 1.0);
  return ldexp(p, static_cast<int>(n));
}

__device__ __forceinline__ double log2_d(double x) {  // x > 0, finite
  int e = 0;
  const double m = frexp(x, &e);
  const double y0 = static_cast<double>(__builtin_amdgcn_logf(static_cast<float>(m)));
  const double r = exp2_d(y0);
  const double y1 = y0 - (r - m) / (r * 0.69314718055994530942);
  return static_cast<double>(e) + y1;
}

// ---------------------------------------------------------------- wave reductions
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Butterfly all-reduce over the 64 lanes: xor 1, xor 2 (quad permutes), half-row
// mirror, row mirror, then the gfx950 permlane16 / permlane32 swaps combine the
// four 16-lane rows.  Every lane ends with the same bits (the ops are commutative).
template <class Op>
__device__ __forceinline__ int wave_allreduce_i(int v, Op op) {
  v = op(v, dpp_i<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_i<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_i<0x141>(v));  // row_half_mirror
  v = op(v, dpp_i<0x140>(v));  // row_mirror
  auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(static_cast<int>(s16[0]), static_cast<int>(s16[1]));
  auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(static_cast<int>(s32[0]), static_cast<int>(s32[1]));
  return v;
}

struct FMaxOp {
  __device__ __forceinline__ int operator()(int a, int b) const {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }
};
struct FAddOp {
  __device__ __forceinline__ int operator()(int a, int b) const {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }
};
struct IMinOp {
  __device__ __forceinline__ int operator()(int a, int b) const { return a < b ? a : b; }
};

__device__ __forceinline__ float wave_max(float v) {
  return __int_as_float(wave_allreduce_i(__float_as_int(v), FMaxOp{}));
}
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(wave_allreduce_i(__float_as_int(v), FAddOp{}));
}
__device__ __forceinline__ int wave_min_i(int v) { return wave_allreduce_i(v, IMinOp{}); }

// fp64 reductions and scans (finalize / sampler kernels, not the streaming loop).
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmax(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    int o = __shfl_xor(v, m, kWave);
    v = o < v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

}  // namespace sv
