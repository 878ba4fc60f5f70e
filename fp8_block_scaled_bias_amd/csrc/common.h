// Shared helpers of the HIP sources: error reporting, argument checks and
// the device-side number-format codecs.  gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

#include "moe_fp8.h"

namespace moe {

// ---- host-side error reporting -------------------------------------------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

#define MOE_REQUIRE(cond, code, ...)        \
  do {                                      \
    if (!(cond)) {                          \
      ::moe::set_error(__VA_ARGS__);        \
      return (code);                        \
    }                                       \
  } while (0)

#define MOE_INVALID(cond, ...) MOE_REQUIRE(cond, MOE_ERR_INVALID, __VA_ARGS__)
#define MOE_UNSUPPORTED(cond, ...) MOE_REQUIRE(cond, MOE_ERR_UNSUPPORTED, __VA_ARGS__)

// Check the launch that was just enqueued.
int check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kWave = 64;

// ---- device-side codecs ----------------------------------------------------

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).  The gfx950
// conversion v_cvt_pk_bf16_f32 was checked bit-identical, over every finite
// fp32 input, to the bit-level rule "add 0x7FFF + lsb, keep the high half".
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return f32x2_to_bf16x2(f, 0.0f) & 0xFFFFu;
}

// fp32 -> OCP E4M3FN codes: round to nearest even, saturate to +-448, keep
// the sign of zero.  Inputs are clamped to [-448, 448] (the sign of zero
// survives the clamp) and converted by v_cvt_pk_fp8_f32, which was checked
// bit-identical, over every fp32 input in [-448, 448], to the format's
// rounding rule: subnormal grid 2^-9 below 2^-6, else 3 mantissa bits with
// round-half-even on the dropped bits.
__device__ __forceinline__ float e4m3_clamp(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}
// two codes in the low 16 bits (a: byte 0, b: byte 1)
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false) & 0xFFFFu;
}
// four codes in one word (a: byte 0 ... d: byte 3)
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) { return f32x2_to_e4m3x2(v, v) & 0xFFu; }

// Lanes 4k..4k+3 of a quad: lane 4k receives the values of lanes 4k+1..4k+3
// (DPP quad_perm; other lanes receive values they do not use).
__device__ __forceinline__ float quad_lane1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x55, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_lane2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xAA, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_lane3(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xFF, 0xF, 0xF, true));
}

// Wave-wide butterfly reductions (wave64).
__device__ __forceinline__ float wave_max_xor(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// SwiGLU backward of one element (fp32): s = 1 / (1 + exp(-g)),
// dg = dh u s (1 + g (1 - s)), du = dh g s, h = g s u.  Every kernel that
// forms these values calls this, so they agree bit for bit.
__device__ __forceinline__ void swiglu_bwd_elem(float g, float u, float d, float* dg, float* du,
                                                float* h) {
  const float s = 1.0f / (1.0f + expf(-g));
  const float gs = g * s;
  *dg = d * u * s * (1.0f + g * (1.0f - s));
  *du = d * gs;
  *h = gs * u;
}

// The quotients x / s of the quantisers with one division per scale instead
// of one per element: with y the correctly rounded 1/s, q = x*y lies within
// an ulp of x/s, the residual x - q*s is exact as one FMA, and q + (x -
// q*s)*y rounded once is the correctly rounded quotient (Markstein's theorem
// on division through a correctly rounded reciprocal), so the codes equal
// those of x / s bit for bit; a zero quotient keeps the sign of x.  This
// needs y finite and no underflow in the residual wherever a code depends on
// the quotient (|x/s| >= 2^-10): scales in [2^-90, 2^100] (recip_ok); the
// quantisers divide for any other scale.
__device__ __forceinline__ bool recip_ok(float s) { return s >= 0x1p-90f && s <= 0x1p100f; }
__device__ __forceinline__ float div_recip(float x, float s, float y) {
  const float q = x * y;
  return copysignf(fmaf(fmaf(-q, s, x), y, q), q);
}

// 1x128 E4M3 quantisation of one tile spread over 16 consecutive lanes (lane
// l % 16 holds elements 8 (l % 16) .. + 7; all 16 lanes must call it
// together): scale = amax / 448 (1 for an all-zero tile), codes = E4M3 of
// v / scale (round to nearest even, saturating).  Returns the lane's 8
// codes; *scale gets the tile's scale.
__device__ __forceinline__ uint2 quant_tile_1x128(const float* v, float* scale) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max_xor(amax, 16);
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  *scale = s;
  if (recip_ok(s)) {
    const float y = 1.0f / s;
    return make_uint2(f32x4_to_e4m3x4(div_recip(v[0], s, y), div_recip(v[1], s, y),
                                      div_recip(v[2], s, y), div_recip(v[3], s, y)),
                      f32x4_to_e4m3x4(div_recip(v[4], s, y), div_recip(v[5], s, y),
                                      div_recip(v[6], s, y), div_recip(v[7], s, y)));
  }
  return make_uint2(f32x4_to_e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s),
                    f32x4_to_e4m3x4(v[4] / s, v[5] / s, v[6] / s, v[7] / s));
}

}  // namespace moe
