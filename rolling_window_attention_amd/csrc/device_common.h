// Device helpers shared by the librfattn kernels (gfx950 only).
//
// * bf16 <-> float conversions on raw 16-bit patterns;
// * the bit-exact 3D-RoPE rotation of one 16-byte chunk (4 rotation pairs);
// * small exact integer division for token -> (frame, row, column).
//
// 3D-RoPE over (time, height, width): "Amazon and Reactor tune Trainium for
// real-time video generation", section "Three problems for generic compilers".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rfattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// cos/sin tables, float2 = (cos, sin) of pos * base^(-j/P), rounded to float32.
struct RopeTables {
  const float2* t;  // [max_frame][pt]
  const float2* h;  // [grid_h][ph]
  const float2* w;  // [grid_w][pw]
  int pt, ph, pw;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two float64 values -> a packed pair of bf16 (low = lo), each rounded to
// nearest even directly (no double rounding).  Each value is first rounded to
// float32 with round-to-odd -- truncated toward zero, and the last bit set when
// that was inexact -- which keeps 16 bits more than bf16, so the second rounding
// (v_cvt_pk_bf16_f32, to nearest even) gives the correctly rounded bf16 of the
// float64 value (rounding to odd with at least two extra bits, then to nearest,
// equals rounding to nearest once).  The float32 rounding of the conversion is
// to nearest; when it went away from zero, one ulp toward zero is its
// truncation.  Finite inputs only.
__device__ __forceinline__ float f64_to_f32_odd(double y) {
  const float f = (float)y;
  const double back = (double)f;
  uint32_t fb = __float_as_uint(f);
  const bool inexact = back != y;
  fb -= (inexact && fabs(back) > fabs(y)) ? 1u : 0u;
  fb |= inexact ? 1u : 0u;
  return __uint_as_float(fb);
}
typedef __bf16 rf_bf16x2 __attribute__((ext_vector_type(2)));
typedef float rf_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f64x2_to_bf16x2(double lo, double hi) {
  const rf_f32x2 f = {f64_to_f32_odd(lo), f64_to_f32_odd(hi)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, rf_bf16x2));
}

// (cos, sin) of rotation pair p for a token at (frame t, row r, column c).
__device__ __forceinline__ float2 rope_cs(const RopeTables& T, int p, int64_t t, int r, int c) {
  const float2* ptr;
  if (p < T.pt) {
    ptr = T.t + t * T.pt + p;
  } else if (p < T.pt + T.ph) {
    ptr = T.h + (int64_t)r * T.ph + (p - T.pt);
  } else {
    ptr = T.w + (int64_t)c * T.pw + (p - T.pt - T.ph);
  }
  return *ptr;
}

// Rotate one 16-byte chunk (8 bf16 = pairs p0..p0+3) of a token at (t, r, c):
//   y0 = bf16(fl64(x0*c - x1*s)),  y1 = bf16(fl64(x0*s + x1*c)).
// bf16*float32 products carry at most 32 significant bits, so they are exact
// in float64; whether the compiler contracts to FMA does not change results.
__device__ __forceinline__ u32x4 rope_chunk(u32x4 x, int p0, int64_t t, int r, int c,
                                            const RopeTables& T) {
  uint32_t in[4] = {x[0], x[1], x[2], x[3]};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float2 cs = rope_cs(T, p0 + k, t, r, c);
    double x0 = (double)bf16_to_f32(in[k] & 0xFFFFu);
    double x1 = (double)bf16_to_f32(in[k] >> 16);
    double cc = (double)cs.x, ss = (double)cs.y;
    double y0 = x0 * cc - x1 * ss;
    double y1 = x0 * ss + x1 * cc;
    out[k] = f64x2_to_bf16x2(y0, y1);
  }
  u32x4 y = {out[0], out[1], out[2], out[3]};
  return y;
}

// As rope_chunk, with the rotated pair scaled by `scale` in float64 before its
// single rounding to bf16 (the attention kernel's pre-scaled query operand).
__device__ __forceinline__ u32x4 rope_chunk_scaled(u32x4 x, int p0, int64_t t, int r, int c,
                                                   const RopeTables& T, double scale) {
  uint32_t in[4] = {x[0], x[1], x[2], x[3]};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float2 cs = rope_cs(T, p0 + k, t, r, c);
    double x0 = (double)bf16_to_f32(in[k] & 0xFFFFu);
    double x1 = (double)bf16_to_f32(in[k] >> 16);
    double cc = (double)cs.x, ss = (double)cs.y;
    double y0 = (x0 * cc - x1 * ss) * scale;
    double y1 = (x0 * ss + x1 * cc) * scale;
    out[k] = f64x2_to_bf16x2(y0, y1);
  }
  u32x4 y = {out[0], out[1], out[2], out[3]};
  return y;
}

// (cos, sin) of the 4 rotation pairs p0..p0+3 of a token at (t, r, c), widened
// to float64 (exactly), for rope_chunk_cs.
struct ChunkCS {
  double c[4], s[4];
};
__device__ __forceinline__ ChunkCS rope_chunk_cs_of(const RopeTables& T, int p0, int64_t t, int r, int c) {
  ChunkCS out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float2 cs = rope_cs(T, p0 + k, t, r, c);
    out.c[k] = (double)cs.x;
    out.s[k] = (double)cs.y;
  }
  return out;
}

// rope_chunk with the chunk's (cos, sin) given: the same arithmetic, so the
// same bits, when several chunks share the pairs and the position (the heads
// of one token).
__device__ __forceinline__ u32x4 rope_chunk_cs(u32x4 x, const ChunkCS& cs) {
  uint32_t in[4] = {x[0], x[1], x[2], x[3]};
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    double x0 = (double)bf16_to_f32(in[k] & 0xFFFFu);
    double x1 = (double)bf16_to_f32(in[k] >> 16);
    double y0 = x0 * cs.c[k] - x1 * cs.s[k];
    double y1 = x0 * cs.s[k] + x1 * cs.c[k];
    out[k] = f64x2_to_bf16x2(y0, y1);
  }
  u32x4 y = {out[0], out[1], out[2], out[3]};
  return y;
}

// Exact unsigned division n / d for n < 2^24, d >= 1: a float estimate is off
// by at most one and is corrected with one multiply-subtract.
__device__ __forceinline__ uint32_t small_div(uint32_t n, uint32_t d, float inv_d, uint32_t* rem) {
  uint32_t q = (uint32_t)((float)n * inv_d);
  int32_t r = (int32_t)(n - q * d);
  if (r < 0) { q -= 1; r += (int32_t)d; }
  if (r >= (int32_t)d) { q += 1; r -= (int32_t)d; }
  *rem = (uint32_t)r;
  return q;
}

}  // namespace rfattn
