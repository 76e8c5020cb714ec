// Device-side helpers shared by the gfx950 kernels: storage codecs, row views
// and wavefront reductions.  Formats: OCP E4M3FN (FP8), BF16, OCP MX E2M1 +
// E8M0 (MXFP4); encoders round to nearest-even and saturate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

constexpr int kWave = 64;

// ------------------------------------------------------------ store view
struct Store {
  const uint8_t* rows;
  const void* scales;
  int64_t cap;
  int dim, rope, fmt, row_bytes;
};

struct StoreW {
  uint8_t* rows;
  void* scales;
  int64_t cap;
  int dim, rope, fmt, row_bytes;
};

inline Store view(const csa_store& s) {
  return Store{(const uint8_t*)s.rows, s.scales, s.cap, s.dim, s.rope_dim, s.fmt, s.row_bytes};
}
inline StoreW wview(const csa_store& s) {
  return StoreW{(uint8_t*)s.rows, s.scales, s.cap, s.dim, s.rope_dim, s.fmt, s.row_bytes};
}

// ------------------------------------------------- RMSNorm / partial RoPE
// Post-processing of stored rows and queries (csa_norm_rope): gain == NULL
// means no RMSNorm, rope_dims == 0 no rotation.
struct NormRope {
  const float* gain;
  float eps;
  int rope_dims;
  const float* theta;
  int64_t pos0;
};
inline NormRope norm_rope_of(const csa_norm_rope* p) {
  return p ? NormRope{p->norm_gain, p->norm_eps, p->rope_dims, p->rope_theta, p->pos0}
           : NormRope{nullptr, 0.0f, 0, nullptr, 0};
}

// sin and cos of a binary32 angle x, to binary32 rounding.  For |x| < 1.6e6:
// Cody-Waite argument reduction (Cody and Waite, "Software Manual for the
// Elementary Functions", 1980) by pi/2 in binary64, pi/2 split into
// P1 + P2 + P3 with P1 and P2 of 33 significant bits (k P1 and k P2 are exact
// for |k| < 2^20), then the Taylor series of sin and cos in binary64 on the
// reduced argument |r| <= pi/4 (terms to r^17 and r^16: truncation error
// below 1e-19).  Larger arguments take sincosf.  (sincosf reduces arguments
// above about 2^15 with a routine that keeps a small array in scratch memory,
// a few memory round trips per call; positions of long contexts reach there.)
__device__ __forceinline__ void sincos_angle(float x, float* s, float* c) {
  if (!(fabsf(x) < 1.6e6f)) {
    sincosf(x, s, c);
    return;
  }
  const double xd = (double)x;
  const double k = rint(xd * 0.6366197723675814);           // nearest multiple of pi/2
  const double r = ((xd - k * 1.5707963267341256) - k * 6.077100506303966e-11) - k * 2.0222662487959506e-21;
  const double r2 = r * r;
  const double sp = r * (1.0 + r2 * (-1.0 / 6 + r2 * (1.0 / 120 + r2 * (-1.0 / 5040 + r2 * (1.0 / 362880 +
                    r2 * (-1.0 / 39916800 + r2 * (1.0 / 6227020800.0 + r2 * (-1.0 / 1307674368000.0 +
                    r2 * (1.0 / 355687428096000.0)))))))));
  const double cp = 1.0 + r2 * (-1.0 / 2 + r2 * (1.0 / 24 + r2 * (-1.0 / 720 + r2 * (1.0 / 40320 +
                    r2 * (-1.0 / 3628800 + r2 * (1.0 / 479001600.0 + r2 * (-1.0 / 87178291200.0 +
                    r2 * (1.0 / 20922789888000.0))))))));
  switch ((int)k & 3) {                                     // x = k pi/2 + r
    case 0: *s = (float)sp; *c = (float)cp; break;
    case 1: *s = (float)cp; *c = (float)-sp; break;
    case 2: *s = (float)-sp; *c = (float)-cp; break;
    default: *s = (float)-cp; *c = (float)sp; break;
  }
}

// Turn the pair (x, y) by the binary32 angle fl32(pos * theta).
__device__ __forceinline__ void rope_pair(float& x, float& y, float pos, float theta) {
  float sn, cs;
  sincos_angle(__fmul_rn(pos, theta), &sn, &cs);
  const float nx = x * cs - y * sn, ny = x * sn + y * cs;
  x = nx;
  y = ny;
}

// ------------------------------------------------------------------ BF16
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// -------------------------------------------------------------- FP8 E4M3FN
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// Round-to-nearest-even E4M3FN code of x, saturating at 448; sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t au = u & 0x7fffffffu;
  if (au > 0x7f800000u) return 0x7fu;                    // NaN
  const float a = __uint_as_float(au);
  if (a >= 448.0f) return s | 0x7eu;
  if (a < 0.015625f) {                                   // below 2^-6: spacing 2^-9
    return s | (uint32_t)rintf(a * 512.0f);              // 8 -> code 0x08 = 2^-6
  }
  uint32_t r = (au + 0x7ffffu + ((au >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
  uint32_t code = r - (120u << 3);
  return s | (code > 0x7eu ? 0x7eu : code);
}

// Smallest power of two s = 2^e with amax <= 448 s; e clamped to [-126, 127];
// amax == 0 gives 1.
__device__ __forceinline__ float fp8_row_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  int a = ilogbf(amax);
  int e = (amax <= ldexpf(448.0f, a - 8)) ? a - 8 : a - 7;
  e = e < -126 ? -126 : (e > 127 ? 127 : e);
  return ldexpf(1.0f, e);
}

// ---------------------------------------------------------------- E2M1
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t mag = c & 7u;
  float v = mag < 4u ? 0.5f * (float)mag : (mag == 4u ? 2.0f : (mag == 5u ? 3.0f : (mag == 6u ? 4.0f : 6.0f)));
  return (c & 8u) ? -v : v;
}

__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const uint32_t s = (__float_as_uint(x) >> 28) & 8u;
  const float a = fabsf(x);
  float q2;  // twice the rounded magnitude
  if (a < 2.0f) q2 = rintf(a * 2.0f);
  else if (a < 4.0f) q2 = 2.0f * rintf(a);
  else q2 = 4.0f * rintf(a * 0.5f);
  q2 = fminf(q2, 12.0f);
  uint32_t qi = (uint32_t)q2;
  uint32_t mag = qi <= 4u ? qi : (qi == 6u ? 5u : (qi == 8u ? 6u : 7u));
  return s | mag;
}

// OCP MX shared exponent of a block: floor(log2 amax) - 2, clamped to
// [-127, 127]; an all-zero block gets -127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = ilogbf(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ------------------------------------------------------- wave reductions
template <int W = kWave>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
  return v;
}
template <int W = kWave>
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
// Map the hardware workgroup index to a logical one so that runs of G
// consecutive logical indices (neighbouring queries, which share most of
// their window rows and many compressed entries) execute on one XCD, while
// the runs themselves are interleaved across XCDs so that the load stays
// balanced when work grows with position.  A permutation of [0, n): each
// block of 8G indices is permuted within itself, a ragged tail is identity.
template <int G = 64>
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t n) {
  constexpr int kXcd = 8;
  const int64_t full = n / (kXcd * G) * (kXcd * G);
  if (i >= full) return i;
  const int64_t x = i % kXcd, j = i / kXcd;
  return (j / G) * (kXcd * G) + x * G + (j % G);
}

// Order-preserving uint32 key of a float score; larger key = larger score.
// -0 is folded into +0 first.  Every finite score maps to a key >= 0x00800000,
// so 0 is free to mark "no entry".
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace csa
