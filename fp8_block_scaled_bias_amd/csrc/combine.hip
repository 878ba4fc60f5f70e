// Weighted combine plus shared expert: y[t] = sum_j w[t,j] * D[inv_perm[t,j]]
// + S[t], fp32 accumulation in slot order, one bf16 rounding at the end
// (news.qq.com/rain/a/20241229A05OQF00, section DeepSeekMoE 架构: the shared
// expert always contributes, routed experts by their gate weight; the
// all-to-all combine of section DualPipe 流水线并行 is this gather on one GPU).
//
// HBM bound: per token k+1 rows of H bf16 in, one row out.  A thread owns 8
// contiguous columns (16 B loads/stores); a 128-thread workgroup covers 1024
// columns of one token (H = 7168 is seven whole workgroups).  The token's k
// row indices and weights are uniform (scalar) loads, and every row's 16 B
// is requested before the first is used, so a thread keeps k + 1 loads in
// flight (the sum is still taken in slot order).
#include "common.h"

namespace moe {
namespace {

constexpr int CB_THREADS = 128;
constexpr int CB_COLS = CB_THREADS * 8;

__device__ __forceinline__ void acc8(float* acc, const uint4& v, float w) {
  const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, bf16_to_f32(x[i] & 0xFFFFu), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, bf16_to_f32(x[i] >> 16), acc[2 * i + 1]);
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// KC > 0: k == KC at compile time; KC == 0: any k in [1, 8]
template <int KC>
__global__ __launch_bounds__(CB_THREADS) void combine_kernel(const uint16_t* __restrict__ D,
                                                             const int32_t* __restrict__ inv_perm,
                                                             const float* __restrict__ w,
                                                             const uint16_t* __restrict__ S,
                                                             int64_t T, int k_rt, int64_t H,
                                                             uint16_t* __restrict__ y) {
  const int k = KC > 0 ? KC : k_rt;
  const int64_t bx = (H + CB_COLS - 1) / CB_COLS;
  const int64_t t = blockIdx.x / bx;
  const int64_t c = ((blockIdx.x - t * bx) * CB_THREADS + threadIdx.x) * 8;
  if (c >= H) return;
  uint4 v[8];
  float wj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      const int64_t r = inv_perm[t * k + j];
      wj[j] = w[t * k + j];
      v[j] = load16(D + r * H + c);
    }
  }
  uint4 sv = {0u, 0u, 0u, 0u};
  if (S) sv = load16(S + t * H + c);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) acc8(acc, v[j], wj[j]);
  if (S) {
    const uint32_t x[4] = {sv.x, sv.y, sv.z, sv.w};
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
  MOE_INVALID(T >= 0 && T * ceil_div(H, CB_COLS) <= 0x7FFFFFFF, "moe_combine: T=%lld too large",
              (long long)T);
  MOE_INVALID(k >= 1 && k <= 8, "moe_combine: k=%d must be in [1, 8]", (int)k);
  MOE_INVALID(H > 0 && H % 8 == 0, "moe_combine: H=%lld must be a positive multiple of 8",
              (long long)H);
  if (T == 0) return MOE_OK;
  MOE_INVALID(expert_out_bf16 && inv_perm && topk_w && y_bf16, "moe_combine: null pointer");
  MOE_INVALID(((uintptr_t)expert_out_bf16 & 15) == 0 && ((uintptr_t)y_bf16 & 15) == 0 &&
                  ((uintptr_t)shared_out_bf16 & 15) == 0,
              "moe_combine: D, S and y must be 16-byte aligned");
  const int64_t bx = ceil_div(H, CB_COLS);
  const dim3 grid((unsigned)(bx * T)), block(CB_THREADS);
  const uint16_t* Dp = static_cast<const uint16_t*>(expert_out_bf16);
  const uint16_t* Sp = static_cast<const uint16_t*>(shared_out_bf16);
  uint16_t* yp = static_cast<uint16_t*>(y_bf16);
  if (k == 8)
    combine_kernel<8><<<grid, block, 0, as_stream(stream)>>>(Dp, inv_perm, topk_w, Sp, T, k, H, yp);
  else
    combine_kernel<0><<<grid, block, 0, as_stream(stream)>>>(Dp, inv_perm, topk_w, Sp, T, k, H, yp);
  return check_launch("moe_combine");
}
