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
//
// Both kernels can also write the 1x128 E4M3 quantisation of their bf16
// gradient rows (the input-gradient GEMM's operand), from the stored bf16
// values with the quantiser's own tile routine: 16 consecutive lanes hold
// one 128-column tile, so the rows are not read back from HBM.
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
    int n_shared, uint16_t* __restrict__ dD, float* __restrict__ dw, uint8_t* __restrict__ dq,
    float* __restrict__ dqs) {
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
      const uint4 ob = f32_to_bf16x8(o);
      *reinterpret_cast<uint4*>(dD + rows[j] * H + c) = ob;
      if (dq) {
        float q[8], s;
        bf16x8_to_f32(ob, q);
        *reinterpret_cast<uint2*>(dq + rows[j] * H + c) = quant_tile_1x128(q, &s);
        if ((tid & 15) == 0) dqs[rows[j] * (H >> 7) + (c >> 7)] = s;
      }
    }
    if (n_shared) {
      *reinterpret_cast<uint4*>(dD + (T * k + t) * H + c) = v;
      if (dq) {
        float s;
        *reinterpret_cast<uint2*>(dq + (T * k + t) * H + c) = quant_tile_1x128(g, &s);
        if ((tid & 15) == 0) dqs[(T * k + t) * (H >> 7) + (c >> 7)] = s;
      }
    }
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
    uint16_t* __restrict__ dgu, uint16_t* __restrict__ h, uint8_t* __restrict__ dq,
    float* __restrict__ dqs) {
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
    for (int i = 0; i < 8; ++i) swiglu_bwd_elem(g[i], u[i], d[i], &dg[i], &du[i], &hv[i]);
    const uint4 dgb = f32_to_bf16x8(dg), dub = f32_to_bf16x8(du);
    *reinterpret_cast<uint4*>(dgu + m * 2 * I + c) = dgb;
    *reinterpret_cast<uint4*>(dgu + m * 2 * I + I + c) = dub;
    *reinterpret_cast<uint4*>(h + m * I + c) = f32_to_bf16x8(hv);
    if (dq) {
      float q[8], s0, s1;
      bf16x8_to_f32(dgb, q);
      *reinterpret_cast<uint2*>(dq + m * 2 * I + c) = quant_tile_1x128(q, &s0);
      bf16x8_to_f32(dub, q);
      *reinterpret_cast<uint2*>(dq + m * 2 * I + I + c) = quant_tile_1x128(q, &s1);
      if ((threadIdx.x & 15) == 0) {
        dqs[m * (I >> 6) + (c >> 7)] = s0;
        dqs[m * (I >> 6) + ((I + c) >> 7)] = s1;
      }
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_combine_backward(const void* dy_bf16, const int32_t* inv_perm,
                                    const float* topk_w, const void* expert_out_bf16, int64_t T,
                                    int32_t k, int64_t H, int32_t n_shared, void* d_expert_out_bf16,
                                    float* d_topk_w, uint8_t* d_expert_out_e4m3,
                                    float* d_expert_out_scale, void* stream) {
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
  MOE_INVALID((d_expert_out_e4m3 == nullptr) == (d_expert_out_scale == nullptr),
              "moe_combine_backward: dD codes and scales are given together or not at all");
  if (d_expert_out_e4m3) {
    MOE_INVALID(H % 128 == 0, "moe_combine_backward: quantised dD needs H %% 128 == 0, got %lld",
                (long long)H);
    MOE_INVALID(((uintptr_t)d_expert_out_e4m3 & 7) == 0 && ((uintptr_t)d_expert_out_scale & 3) == 0,
                "moe_combine_backward: dD codes must be 8-byte, scales 4-byte aligned");
  }
  combine_backward_kernel<8><<<dim3((unsigned)T), dim3(CB), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(dy_bf16), inv_perm, topk_w,
      static_cast<const uint16_t*>(expert_out_bf16), T, k, H, n_shared,
      static_cast<uint16_t*>(d_expert_out_bf16), d_topk_w, d_expert_out_e4m3, d_expert_out_scale);
  return check_launch("moe_combine_backward");
}

extern "C" int swiglu_backward(const void* gu_bf16, const void* dh_bf16, int64_t M, int64_t I,
                               void* dgu_bf16, void* h_bf16, uint8_t* dgu_e4m3, float* dgu_scale,
                               void* stream) {
  clear_error();
  MOE_INVALID(M >= 0, "swiglu_backward: M=%lld < 0", (long long)M);
  MOE_INVALID(I > 0 && I % 8 == 0, "swiglu_backward: I=%lld must be a positive multiple of 8",
              (long long)I);
  if (M == 0) return MOE_OK;
  MOE_INVALID(gu_bf16 && dh_bf16 && dgu_bf16 && h_bf16, "swiglu_backward: null pointer");
  MOE_INVALID(((uintptr_t)gu_bf16 & 15) == 0 && ((uintptr_t)dh_bf16 & 15) == 0 &&
                  ((uintptr_t)dgu_bf16 & 15) == 0 && ((uintptr_t)h_bf16 & 15) == 0,
              "swiglu_backward: all tensors must be 16-byte aligned");
  MOE_INVALID((dgu_e4m3 == nullptr) == (dgu_scale == nullptr),
              "swiglu_backward: dGU codes and scales are given together or not at all");
  if (dgu_e4m3) {
    MOE_INVALID(I % 128 == 0, "swiglu_backward: quantised dGU needs I %% 128 == 0, got %lld",
                (long long)I);
    MOE_INVALID(((uintptr_t)dgu_e4m3 & 7) == 0 && ((uintptr_t)dgu_scale & 3) == 0,
                "swiglu_backward: dGU codes must be 8-byte, scales 4-byte aligned");
  }
  const int64_t n = M * (I / 8);
  const int64_t blocks = std::min<int64_t>(ceil_div(n, 256), 256 * 64);
  swiglu_backward_kernel<<<dim3((unsigned)blocks), dim3(256), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(gu_bf16), static_cast<const uint16_t*>(dh_bf16), M, I,
      static_cast<uint16_t*>(dgu_bf16), static_cast<uint16_t*>(h_bf16), dgu_e4m3, dgu_scale);
  return check_launch("swiglu_backward");
}

// ---- router backward -----------------------------------------------------------
// The gate weights are w_j = s_j / S over a token's k selected experts,
// s_j = sigmoid(x . C[e_j]) (unbiased scores; the selection and the bias
// carry no gradient: the bias only selects, news.qq.com article section
// 无额外损耗的负载均衡; gating stays in FP32, section FP8 低精度训练), S = sum s_j:
//   dlogit_j = (dw_j - sum_i dw_i w_i) / S * s_j (1 - s_j)
//   dx[t]    = dx_in[t] + sum_j dlogit_j C[e_j]
//   dC[e]    = sum over the rows r of expert e of dlogit(r) x[token(r)]
// The logits are recomputed here in fp32 (one workgroup per token, fixed
// summation order); dlogit is written in expert-row order (through
// inv_perm) for the centroid gradient, which sums each expert's rows in
// row order (one workgroup per expert and 2048 columns).
namespace moe {
namespace {

constexpr int RB = 256;

template <int KMAX>
__global__ __launch_bounds__(RB) void router_backward_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ C, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, const int32_t* __restrict__ inv_perm,
    const uint16_t* __restrict__ dx_in, int64_t T, int64_t H, int E, int k,
    uint16_t* __restrict__ dx_out, float* __restrict__ dlogit_rows,
    const float* __restrict__ topk_s) {
  __shared__ float s_part[RB / 64][KMAX];
  __shared__ float s_dl[KMAX];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t e[KMAX];
  float dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    // ids outside [0, E) (not produced by the router) read expert E - 1
    e[j] = j < k ? (int64_t)min((uint32_t)idx[t * k + j], (uint32_t)(E - 1)) : 0;
    dot[j] = 0.0f;
  }
  const uint16_t* xr = x + t * H;
  // without the forward's scores, the selected experts' logits again
  for (int64_t c = topk_s ? H : (int64_t)tid * 8; c < H; c += RB * 8) {
    float xv[8];
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(xr + c), xv);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      const float4 c0 = *reinterpret_cast<const float4*>(C + e[j] * H + c);
      const float4 c1 = *reinterpret_cast<const float4*>(C + e[j] * H + c + 4);
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) dot[j] = fmaf(xv[i], cv[i], dot[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float v = dot[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) s_part[wv][j] = v;
  }
  __syncthreads();
  if (tid == 0) {
    float s[KMAX], S = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      if (topk_s) {
        s[j] = topk_s[t * k + j];
      } else {
        const float l = (s_part[0][j] + s_part[1][j]) + (s_part[2][j] + s_part[3][j]);
        s[j] = 1.0f / (1.0f + expf(-l));
      }
      S += s[j];
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      m = fmaf(dw[t * k + j], s[j] / S, m);
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      const float dl = (dw[t * k + j] - m) / S * s[j] * (1.0f - s[j]);
      s_dl[j] = dl;
      // rows outside [0, T*k) (not produced by the permutation) are skipped
      const uint32_t row = (uint32_t)inv_perm[t * k + j];
      if (row < (uint32_t)(T * k)) dlogit_rows[row] = dl;
    }
  }
  __syncthreads();
  float dl[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) dl[j] = j < k ? s_dl[j] : 0.0f;
  for (int64_t c = (int64_t)tid * 8; c < H; c += RB * 8) {
    float o[8];
    if (dx_in) bf16x8_to_f32(*reinterpret_cast<const uint4*>(dx_in + t * H + c), o);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j >= k) break;
      const float4 c0 = *reinterpret_cast<const float4*>(C + e[j] * H + c);
      const float4 c1 = *reinterpret_cast<const float4*>(C + e[j] * H + c + 4);
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(dl[j], cv[i], o[i]);
    }
    *reinterpret_cast<uint4*>(dx_out + t * H + c) = f32_to_bf16x8(o);
  }
}

constexpr int DC_COLS = RB * 8;

__global__ __launch_bounds__(RB) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * RB + threadIdx.x; i < n; i += (int64_t)gridDim.x * RB)
    p[i] = 0.0f;
}

__global__ __launch_bounds__(RB) void router_dcentroids_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ perm_src,
    const int32_t* __restrict__ offs, const float* __restrict__ dlogit_rows, int64_t T, int64_t H,
    float* __restrict__ dC) {
  const int e = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * DC_COLS + threadIdx.x * 8;
  if (c >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int r0 = offs[e], r1 = offs[e + 1];
  for (int r = r0; r < r1; ++r) {
    const float d = dlogit_rows[r];
    float xv[8];
    // token ids outside [0, T) (not produced by the permutation) read token T - 1
    const int64_t tok = min((uint32_t)perm_src[r], (uint32_t)(T - 1));
    bf16x8_to_f32(*reinterpret_cast<const uint4*>(x + tok * H + c), xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(d, xv[i], acc[i]);
  }
  float* o = dC + (int64_t)e * H + c;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

}  // namespace
}  // namespace moe

extern "C" int moe_router_backward(const void* x_bf16, const float* centroids,
                                   const int32_t* topk_idx, const float* d_topk_w,
                                   const int32_t* inv_perm, const void* dx_in_bf16, int64_t T,
                                   int64_t H, int32_t E, int32_t k, void* dx_out_bf16,
                                   float* dlogit_rows, const float* topk_s, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && T < (1ll << 31), "moe_router_backward: T=%lld out of range", (long long)T);
  MOE_INVALID(k >= 1 && k <= 8, "moe_router_backward: k=%d must be in [1, 8]", (int)k);
  MOE_INVALID(E >= k, "moe_router_backward: E=%d < k", (int)E);
  MOE_INVALID(H > 0 && H % 8 == 0, "moe_router_backward: H=%lld must be a positive multiple of 8",
              (long long)H);
  if (T == 0) return MOE_OK;
  MOE_INVALID(x_bf16 && centroids && topk_idx && d_topk_w && inv_perm && dx_out_bf16 && dlogit_rows,
              "moe_router_backward: null pointer");
  MOE_INVALID(((uintptr_t)x_bf16 & 15) == 0 && ((uintptr_t)centroids & 15) == 0 &&
                  ((uintptr_t)dx_out_bf16 & 15) == 0 && ((uintptr_t)dx_in_bf16 & 15) == 0,
              "moe_router_backward: x, centroids, dx_in and dx_out must be 16-byte aligned");
  MOE_INVALID(((uintptr_t)topk_s & 3) == 0, "moe_router_backward: topk_s must be 4-byte aligned");
  router_backward_kernel<8><<<dim3((unsigned)T), dim3(RB), 0, as_stream(stream)>>>(
      static_cast<const uint16_t*>(x_bf16), centroids, topk_idx, d_topk_w, inv_perm,
      static_cast<const uint16_t*>(dx_in_bf16), T, H, E, k, static_cast<uint16_t*>(dx_out_bf16),
      dlogit_rows, topk_s);
  return check_launch("moe_router_backward");
}

extern "C" int moe_router_dcentroids(const void* x_bf16, const int32_t* perm_src,
                                     const int32_t* group_offsets, const float* dlogit_rows,
                                     int64_t T, int64_t H, int32_t E, float* d_centroids,
                                     void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && T < (1ll << 31), "moe_router_dcentroids: T=%lld out of range", (long long)T);
  MOE_INVALID(E >= 1 && E <= 65535, "moe_router_dcentroids: E=%d out of [1, 65535]", (int)E);
  MOE_INVALID(H > 0 && H % 8 == 0, "moe_router_dcentroids: H=%lld must be a positive multiple of 8",
              (long long)H);
  MOE_INVALID(d_centroids && ((uintptr_t)d_centroids & 15) == 0,
              "moe_router_dcentroids: d_centroids must be non-null and 16-byte aligned");
  if (T == 0) {  // no rows: the gradient is zero
    zero_f32_kernel<<<dim3(256), dim3(RB), 0, as_stream(stream)>>>(d_centroids, (int64_t)E * H);
    return check_launch("moe_router_dcentroids(zero)");
  }
  MOE_INVALID(x_bf16 && perm_src && group_offsets && dlogit_rows,
              "moe_router_dcentroids: null pointer");
  MOE_INVALID(((uintptr_t)x_bf16 & 15) == 0 && ((uintptr_t)d_centroids & 15) == 0,
              "moe_router_dcentroids: x and d_centroids must be 16-byte aligned");
  router_dcentroids_kernel<<<dim3((unsigned)ceil_div(H, DC_COLS), (unsigned)E), dim3(RB), 0,
                             as_stream(stream)>>>(static_cast<const uint16_t*>(x_bf16), perm_src,
                                                  group_offsets, dlogit_rows, T, H, d_centroids);
  return check_launch("moe_router_dcentroids");
}
