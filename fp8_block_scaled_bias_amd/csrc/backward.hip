// Elementwise steps of the expert path's backward (news.qq.com/rain/a/
// 20241229A05OQF00: section DeepSeekMoE 架构 for the gate-weighted combine
// with an always-on shared expert, section 工程 › DualPipe 流水线并行 for the
// backward-for-input / backward-for-weights split of a chunk).
//
// combine backward: the forward y[t] = sum_j w[t,j] D[r(t,j)] + D[shared t]
// gives dD[r(t,j)] = w[t,j] dy[t] (stored as bf16 of the fp32 product),
// dD[shared t] = dy[t] and dw[t,j] = <dy[t], D[r(t,j)]> (fp32).  One
// workgroup per token; 16 B vectors; the dot products are summed per thread
// in column order, then over the block in a fixed tree (deterministic).
//
// SwiGLU backward: from the bf16 gate/up outputs g, u and dh,
//   s = 1 / (1 + exp(-g)),  dg = dh u s (1 + g (1 - s)),  du = dh g s,
// plus h = g s u (the down projection's weight-gradient operand), in fp32,
// stored as bf16.  HBM bound, grid-stride over 8-element vectors.
#include "common.h"

namespace moe {
namespace {

constexpr int CB = 256;

__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}
__device__ __forceinline__ uint4 f32_to_bf16x8(const float* f) {
  return make_uint4(f32x2_to_bf16x2(f[0], f[1]), f32x2_to_bf16x2(f[2], f[3]),
                    f32x2_to_bf16x2(f[4], f[5]), f32x2_to_bf16x2(f[6], f[7]));
}

template <int KMAX>
__global__ __launch_bounds__(CB) void combine_backward_kernel(
    const uint16_t* __restrict__ dy, const int32_t* __restrict__ inv_perm,
    const float* __restrict__ w, const uint16_t* __restrict__ D, int64_t T, int k, int64_t H,
    int n_shared, uint16_t* __restrict__ dD, float* __restrict__ dw) {
  __shared__ float s_dot[CB / 64][KMAX];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t rows[KMAX];
  float wt[KMAX], dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = j < k ? inv_perm[t * k + j] : 0;
    wt[j] = j < k ? w[t * k + j] : 0.0f;
    dot[j] = 0.0f;
  }
  const uint16_t* dyr = dy + t * H;
  for (int64_t c = (int64_t)tid * 8; c < H; c += CB * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(dyr + c);
    float g[8];
    bf16x8_to_f32(v, g);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      float d[8], o[8];
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(D + rows[j] * H + c), d);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot[j] = fmaf(g[i], d[i], dot[j]);
        o[i] = wt[j] * g[i];
      }
      *reinterpret_cast<uint4*>(dD + rows[j] * H + c) = f32_to_bf16x8(o);
    }
    if (n_shared) *reinterpret_cast<uint4*>(dD + (T * k + t) * H + c) = v;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float v = dot[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) s_dot[wv][j] = v;
  }
  __syncthreads();
  if (tid < k) dw[t * k + tid] = (s_dot[0][tid] + s_dot[1][tid]) + (s_dot[2][tid] + s_dot[3][tid]);
}

__global__ __launch_bounds__(256) void swiglu_backward_kernel(
    const uint16_t* __restrict__ gu, const uint16_t* __restrict__ dh, int64_t M, int64_t I,
    uint16_t* __restrict__ dgu, uint16_t* __restrict__ h) {
  const int64_t per_row = I >> 3;
  const int64_t n = M * per_row;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < n;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = p / per_row, c = (p - m * per_row) * 8;
    float g[8], u[8], d[8], dg[8], du[8], hv[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(gu + m * 2 * I + c), g);
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(gu + m * 2 * I + I + c), u);
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(dh + m * I + c), d);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = 1.0f / (1.0f + expf(-g[i]));
      const float gs = g[i] * s;
      dg[i] = d[i] * u[i] * s * (1.0f + g[i] * (1.0f - s));
      du[i] = d[i] * gs;
      hv[i] = gs * u[i];
    }
    *reinterpret_cast<uint4*>(dgu + m * 2 * I + c) = f32_to_bf16x8(dg);
    *reinterpret_cast<uint4*>(dgu + m * 2 * I + I + c) = f32_to_bf16x8(du);
    *reinterpret_cast<uint4*>(h + m * I + c) = f32_to_bf16x8(hv);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine_backward(const void* dy_bf16, const int32_t* inv_perm,
                                    const float* topk_w, const void* expert_out_bf16, int64_t T,
                                    int32_t k, int64_t H, int32_t n_shared, void* d_expert_out_bf16,
                                    float* d_topk_w, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && T < (1ll << 31), "moe_combine_backward: T=%lld out of range", (long long)T);
  MOE_INVALID(k >= 1 && k <= 8, "moe_combine_backward: k=%d must be in [1, 8]", (int)k);
  MOE_INVALID(H > 0 && H % 8 == 0, "moe_combine_backward: H=%lld must be a positive multiple of 8",
              (long long)H);
  MOE_INVALID(n_shared == 0 || n_shared == 1, "moe_combine_backward: n_shared=%d must be 0 or 1",
              (int)n_shared);
  if (T == 0) return MOE_OK;
  MOE_INVALID(dy_bf16 && inv_perm && topk_w && expert_out_bf16 && d_expert_out_bf16 && d_topk_w,
              "moe_combine_backward: null pointer");
  MOE_INVALID(((uintptr_t)dy_bf16 & 15) == 0 && ((uintptr_t)expert_out_bf16 & 15) == 0 &&
                  ((uintptr_t)d_expert_out_bf16 & 15) == 0,
              "moe_combine_backward: dy, D and dD must be 16-byte aligned");
  MOE_INVALID(d_expert_out_bf16 != expert_out_bf16, "moe_combine_backward: dD must not alias D");
  combine_backward_kernel<8><<<dim3((unsigned)T), dim3(CB), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(dy_bf16), inv_perm, topk_w,
      static_cast<const uint16_t*>(expert_out_bf16), T, k, H, n_shared,
      static_cast<uint16_t*>(d_expert_out_bf16), d_topk_w);
  return check_launch("moe_combine_backward");
}

extern "C" int swiglu_backward(const void* gu_bf16, const void* dh_bf16, int64_t M, int64_t I,
                               void* dgu_bf16, void* h_bf16, void* stream) {
  clear_error();
  MOE_INVALID(M >= 0, "swiglu_backward: M=%lld < 0", (long long)M);
  MOE_INVALID(I > 0 && I % 8 == 0, "swiglu_backward: I=%lld must be a positive multiple of 8",
              (long long)I);
  if (M == 0) return MOE_OK;
  MOE_INVALID(gu_bf16 && dh_bf16 && dgu_bf16 && h_bf16, "swiglu_backward: null pointer");
  MOE_INVALID(((uintptr_t)gu_bf16 & 15) == 0 && ((uintptr_t)dh_bf16 & 15) == 0 &&
                  ((uintptr_t)dgu_bf16 & 15) == 0 && ((uintptr_t)h_bf16 & 15) == 0,
              "swiglu_backward: all tensors must be 16-byte aligned");
  const int64_t n = M * (I / 8);
  const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), 256 * 64);
  swiglu_backward_kernel<<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(gu_bf16), static_cast<const uint16_t*>(dh_bf16), M, I,
      static_cast<uint16_t*>(dgu_bf16), static_cast<uint16_t*>(h_bf16));
  return check_launch("swiglu_backward");
}
