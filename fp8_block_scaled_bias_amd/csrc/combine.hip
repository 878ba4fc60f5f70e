// Weighted combine plus shared expert: y[t] = sum_j w[t,j] * D[inv_perm[t,j]]
// + S[t], fp32 accumulation in slot order, one bf16 rounding at the end
// (news.qq.com/rain/a/20241229A05OQF00, section DeepSeekMoE 架构: the shared
// expert always contributes, routed experts by their gate weight; the
// all-to-all combine of section DualPipe 流水线并行 is this gather on one GPU).
//
// HBM bound: per token k+1 rows of H bf16 in, one row out.  A thread owns 8
// contiguous columns (16 B loads/stores); a 256-thread workgroup covers 2048
// columns of one token; the k row indices and weights are uniform loads.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ void acc8(float* acc, const uint4& v, float w) {
  const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, bf16_to_f32(x[i] & 0xFFFFu), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, bf16_to_f32(x[i] >> 16), acc[2 * i + 1]);
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ D,
                                                      const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ S, int64_t T,
                                                      int k, int64_t H, uint16_t* __restrict__ y) {
  const int64_t bx = (H + 2047) / 2048;
  const int64_t t = blockIdx.x / bx;
  const int64_t c = ((blockIdx.x - t * bx) * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int64_t r = inv_perm[t * k + j];
    const float wj = w[t * k + j];
    const uint4 v = *reinterpret_cast<const uint4*>(D + r * H + c);
    acc8(acc, v, wj);
  }
  if (S) {
    const uint4 v = *reinterpret_cast<const uint4*>(S + t * H + c);
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(x[i] & 0xFFFFu);
      acc[2 * i + 1] += bf16_to_f32(x[i] >> 16);
    }
  }
  uint4 o;
  o.x = f32x2_to_bf16x2(acc[0], acc[1]);
  o.y = f32x2_to_bf16x2(acc[2], acc[3]);
  o.z = f32x2_to_bf16x2(acc[4], acc[5]);
  o.w = f32x2_to_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(y + t * H + c) = o;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine(const void* expert_out_bf16, const int32_t* inv_perm,
                           const float* topk_w, const void* shared_out_bf16, int64_t T, int32_t k,
                           int64_t H, void* y_bf16, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && T * ceil_div(H, 2048) <= 0x7FFFFFFF, "moe_combine: T=%lld too large",
              (long long)T);
  MOE_INVALID(k >= 1 && k <= 8, "moe_combine: k=%d must be in [1, 8]", (int)k);
  MOE_INVALID(H > 0 && H % 8 == 0, "moe_combine: H=%lld must be a positive multiple of 8",
              (long long)H);
  if (T == 0) return MOE_OK;
  MOE_INVALID(expert_out_bf16 && inv_perm && topk_w && y_bf16, "moe_combine: null pointer");
  MOE_INVALID(((uintptr_t)expert_out_bf16 & 15) == 0 && ((uintptr_t)y_bf16 & 15) == 0 &&
                  ((uintptr_t)shared_out_bf16 & 15) == 0,
              "moe_combine: D, S and y must be 16-byte aligned");
  const int64_t bx = ceil_div(H, 256 * 8);
  combine_kernel<<<dim3((unsigned)(bx * T)), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(expert_out_bf16), inv_perm, topk_w,
      static_cast<const uint16_t*>(shared_out_bf16), T, k, H, static_cast<uint16_t*>(y_bf16));
  return check_launch("moe_combine");
}
