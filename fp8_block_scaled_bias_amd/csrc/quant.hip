// Fine-grained FP8 quantisation: 1x128 activation tiles (plain or fused
// SwiGLU) and 128x128 weight blocks.
//
// Scale rule (the pages give the granularity only - news.qq.com/rain/a/
// 20241229A05OQF00, section FP8 低精度训练 › 细粒度量化): s = amax / 448 in
// fp32 (1 for an all-zero tile); each element is divided by s and encoded
// to E4M3FN with round-to-nearest-even and saturation.
//
// 1x128 layout: 16 lanes own one 128-element tile, 8 contiguous bf16 (16 B)
// per lane, so a wave reads 4 consecutive tiles = 1 KB of one row
// contiguously; the tile amax is a 4-step butterfly inside the 16 lanes.
// HBM bound: 2 B in + 1 B out per element (+4 B per 128 for the scale).
#include "common.h"

namespace moe {
namespace {

template <int MODE>
__global__ __launch_bounds__(256) void quant_1x128_kernel(
    const uint16_t* __restrict__ in, int64_t K, int64_t ld_in,
    uint8_t* __restrict__ out, float* __restrict__ scales, int64_t n_tiles) {
  const int l16 = threadIdx.x & 15;
  const int64_t tpr = K >> 7;  // tiles per row
  for (int64_t tile = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); tile < n_tiles;
       tile += (int64_t)gridDim.x * 16) {
    const int64_t row = tile / tpr;
    const int64_t tc = tile - row * tpr;
    const uint16_t* src = in + row * ld_in + tc * 128 + l16 * 8;
    float v[8];
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    if (MODE == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(aw[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(aw[i] >> 16);
      }
    } else {
      const uint4 b = *reinterpret_cast<const uint4*>(src + K);
      const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float g = bf16_to_f32(h ? (aw[i] >> 16) : (aw[i] & 0xFFFFu));
          const float u = bf16_to_f32(h ? (bw[i] >> 16) : (bw[i] & 0xFFFFu));
          const float t = expf(-g);
          const float d = 1.0f + t;
          const float sg = g / d;
          v[2 * i + h] = sg * u;
        }
      }
    }
    float s;
    *reinterpret_cast<uint2*>(out + row * K + tc * 128 + l16 * 8) = quant_tile_1x128(v, &s);
    if (l16 == 0) scales[row * tpr + tc] = s;
  }
}

// One workgroup per 128x128 block of one group's [N, K] fp32 matrix.
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const float* __restrict__ w, int64_t N, int64_t K,
    uint8_t* __restrict__ out, float* __restrict__ scales) {
  const int64_t nkb = K >> 7;
  const int64_t kb = blockIdx.x;
  const int64_t nb = blockIdx.y;
  const int64_t g = blockIdx.z;
  const float* base = w + (g * N + nb * 128) * K + kb * 128;
  uint8_t* obase = out + (g * N + nb * 128) * K + kb * 128;
  // thread layout: 32 threads per row (4 floats each), 8 rows per pass; the
  // block stays in registers (16 float4 per thread) between the maximum and
  // the codes, so it is read from memory once
  const int c4 = (threadIdx.x & 31) * 4;
  const int r0 = threadIdx.x >> 5;
  typedef float f4v __attribute__((ext_vector_type(4)));
  f4v v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(base + (int64_t)(r0 + 8 * i) * K + c4));
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  amax = wave_max_xor(amax, 64);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  auto emit = [&](auto dv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<uint32_t*>(obase + (int64_t)(r0 + 8 * i) * K + c4) =
          f32x4_to_e4m3x4(dv(v[i].x), dv(v[i].y), dv(v[i].z), dv(v[i].w));
  };
  if (recip_ok(s)) {
    const float y = 1.0f / s;
    emit([&](float x) { return div_recip(x, s, y); });
  } else {
    emit([&](float x) { return x / s; });
  }
  if (threadIdx.x == 0) scales[(g * (N >> 7) + nb) * nkb + kb] = s;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int fp8_quant_1x128(const void* in_bf16, int64_t M, int64_t K, int64_t ld_in,
                               int32_t mode, uint8_t* out_e4m3, float* scales,
                               void* stream) {
  clear_error();
  MOE_INVALID(M >= 0, "fp8_quant_1x128: M=%lld < 0", (long long)M);
  MOE_INVALID(K > 0 && K % 128 == 0, "fp8_quant_1x128: K=%lld must be a positive multiple of 128",
              (long long)K);
  MOE_INVALID(mode == 0 || mode == 1, "fp8_quant_1x128: mode=%d must be 0 or 1", (int)mode);
  MOE_INVALID(ld_in % 8 == 0 && ld_in >= (mode ? 2 * K : K),
              "fp8_quant_1x128: ld_in=%lld must be a multiple of 8 and >= %lld",
              (long long)ld_in, (long long)(mode ? 2 * K : K));
  if (M == 0) return MOE_OK;
  MOE_INVALID(in_bf16 && out_e4m3 && scales, "fp8_quant_1x128: null pointer");
  MOE_INVALID(((uintptr_t)in_bf16 & 15) == 0 && ((uintptr_t)out_e4m3 & 7) == 0 &&
                  ((uintptr_t)scales & 3) == 0,
              "fp8_quant_1x128: in must be 16-byte, out 8-byte, scales 4-byte aligned");
  const int64_t n_tiles = M * (K / 128);
  const int64_t blocks = std::min<int64_t>(ceil_div(n_tiles, 16), 256 * 64);
  auto* in = static_cast<const uint16_t*>(in_bf16);
  if (mode == 0)
    quant_1x128_kernel<0><<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(
        in, K, ld_in, out_e4m3, scales, n_tiles);
  else
    quant_1x128_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(
        in, K, ld_in, out_e4m3, scales, n_tiles);
  return check_launch("fp8_quant_1x128");
}

extern "C" int fp8_quant_128x128(const float* w_f32, int64_t G, int64_t N, int64_t K,
                                 uint8_t* out_e4m3, float* scales, void* stream) {
  clear_error();
  MOE_INVALID(G >= 0 && G <= 65535, "fp8_quant_128x128: G=%lld out of [0, 65535]", (long long)G);
  MOE_INVALID(N > 0 && N % 128 == 0 && K > 0 && K % 128 == 0,
              "fp8_quant_128x128: N=%lld and K=%lld must be positive multiples of 128",
              (long long)N, (long long)K);
  MOE_INVALID(N / 128 <= 65535 && K / 128 <= (1ll << 31) - 1, "fp8_quant_128x128: too large");
  if (G == 0) return MOE_OK;
  MOE_INVALID(w_f32 && out_e4m3 && scales, "fp8_quant_128x128: null pointer");
  MOE_INVALID(((uintptr_t)w_f32 & 15) == 0 && ((uintptr_t)out_e4m3 & 3) == 0,
              "fp8_quant_128x128: w must be 16-byte and out 4-byte aligned");
  quant_128x128_kernel<<<dim3((unsigned)(K / 128), (unsigned)(N / 128), (unsigned)G), dim3(256), 0,
                         as_stream(stream)>>>(w_f32, N, K, out_e4m3, scales);
  return check_launch("fp8_quant_128x128");
}
