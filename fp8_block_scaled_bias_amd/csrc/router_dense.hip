// The router's backward when the loss also holds the sequence-wise balance
// term: the logits' gradient is then dense over every routed expert.
//
// Method: news.qq.com/rain/a/20241229A05OQF00, section 无额外损耗的负载均衡
// (the bias only selects and has no gradient; the sequence-level balance
// factor alpha = 0.0001) and section FP8 低精度训练 (the gating stays in
// FP32); m.jxzklqfsx.com/aigc/3586.html, section （二）無輔助損失負載均衡策略革新
// (the sequence-level term).  With the selection held fixed (f counts it),
// for token t of sequence b (L_b tokens), scores s of every expert, S = sum_e s:
//   balance: dlogit[t, e] = alpha / L_b * (f[b, e] - sum_i f[b, i] s_i / S) / S
//                           * s_e (1 - s_e)
//   gate:    + (dw_j - sum_i dw_i w_i) / S_sel * s_j (1 - s_j) on the chosen
//            experts e_j, with S_sel = sum_j s_j and w_j = s_j / S_sel
//   dx[t, :] = dx_in[t, :] + sum_e dlogit[t, e] C[e, :]
//   dC[e, :] = sum_t dlogit[t, e] x[t, :]
// The scores are the forward router's fp32 ones (moe_route_scores).
//
// Kernels:
//  1. dense_dlogit: one wave per token, lane l owns experts 4l..4l+3; the
//     two reductions are wave butterflies (fixed order);
//  2. dense_dx: an fp32 GEMM [T, E] x [E, H] plus dx_in, 128 x 128 output
//     tiles, 16-deep K steps through LDS (K-major tiles), 8 x 8 outputs per
//     thread, the next K step's loads in registers during the current one;
//  3. dense_dc: the same GEMM shape for dlogit^T x over a slice of the
//     tokens (x converted from bf16 on the way into LDS), each slice's
//     partial written separately, then
//  4. dc_reduce adds the slices in order.
#include "common.h"

namespace moe {
namespace {

constexpr int DT = 256;   // threads
constexpr int DM = 128;   // output tile rows
constexpr int DN = 128;   // output tile columns
constexpr int DK = 16;    // K step
constexpr int DP = DM + 4;  // LDS row pitch (floats) of the K-major tiles

__global__ __launch_bounds__(DT) void dense_dlogit_kernel(
    const float* __restrict__ scores, const float* __restrict__ ssum,
    const float* __restrict__ seq_f, const int32_t* __restrict__ idx,
    const float* __restrict__ dw, int64_t T, int E, int k, int64_t L, float alpha,
    float* __restrict__ dlogit) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (DT / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int e0 = lane * 4;
  const bool active = e0 < E;
  const int64_t b = t / L;
  const float Lb = (float)min(L, T - b * L);
  float s[4] = {0.f, 0.f, 0.f, 0.f}, f[4] = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const float4 sv = *reinterpret_cast<const float4*>(scores + t * E + e0);
    const float4 fv = *reinterpret_cast<const float4*>(seq_f + b * E + e0);
    s[0] = sv.x; s[1] = sv.y; s[2] = sv.z; s[3] = sv.w;
    f[0] = fv.x; f[1] = fv.y; f[2] = fv.z; f[3] = fv.w;
  }
  const float S = ssum[t];
  float m = (f[0] * s[0] + f[1] * s[1]) + (f[2] * s[2] + f[3] * s[3]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m += __shfl_xor(m, o, 64);
  m = m / S;
  const float c = alpha / Lb;
  float g[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) g[i] = c * (f[i] - m) / S * s[i] * (1.0f - s[i]);
  // the gate part on the chosen experts (every lane computes it)
  float sj[8], dwj[8];
  int ej[8];
  float Ssel = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      ej[j] = (int)min((uint32_t)idx[t * k + j], (uint32_t)(E - 1));  // ids past E: E - 1
      sj[j] = scores[t * E + ej[j]];
      dwj[j] = dw[t * k + j];
      Ssel += sj[j];
    }
  }
  float mg = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) mg = fmaf(dwj[j], sj[j] / Ssel, mg);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k && (ej[j] >> 2) == lane) {
      const float dl = (dwj[j] - mg) / Ssel * sj[j] * (1.0f - sj[j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((ej[j] & 3) == i) g[i] += dl;
    }
  }
  if (active)
    *reinterpret_cast<float4*>(dlogit + t * E + e0) = make_float4(g[0], g[1], g[2], g[3]);
}

// One K step of the 128 x 128 tile: thread (ty, tx) = (tid / 16, tid % 16)
// owns rows 8ty.. and columns 8tx.. of the tile.
__device__ __forceinline__ void tile_step(const float (*As)[DP], const float (*Bs)[DP], int ty,
                                          int tx, float (&acc)[8][8]) {
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) {
    const float4 a0 = *reinterpret_cast<const float4*>(&As[kk][8 * ty]);
    const float4 a1 = *reinterpret_cast<const float4*>(&As[kk][8 * ty + 4]);
    const float4 b0 = *reinterpret_cast<const float4*>(&Bs[kk][8 * tx]);
    const float4 b1 = *reinterpret_cast<const float4*>(&Bs[kk][8 * tx + 4]);
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
  }
}

// dx_out[t, h] = bf16(dx_in[t, h] + sum_e dlogit[t, e] C[e, h]); grid
// (H / 128, ceil(T / 128)).  A = dlogit rows (E contiguous), B = C rows.
__global__ __launch_bounds__(DT) void dense_dx_kernel(
    const float* __restrict__ D, const float* __restrict__ C, const uint16_t* __restrict__ dx_in,
    int64_t T, int64_t H, int E, uint16_t* __restrict__ dx_out) {
  __shared__ __attribute__((aligned(16))) float As[DK][DP];
  __shared__ __attribute__((aligned(16))) float Bs[DK][DP];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t n0 = (int64_t)blockIdx.x * DN, m0 = (int64_t)blockIdx.y * DM;
  // A loads: rows tid/4 and 64 + tid/4, K elements 4 (tid % 4) .. +3
  const int ar = tid >> 2, ak = (tid & 3) * 4;
  // B loads: K row tid/16, columns 8 (tid % 16) .. +7
  const int bk = tid >> 4, bn = (tid & 15) * 8;
  float4 ra0, ra1, rb0, rb1;
  auto load = [&](int k0) {
    const int64_t r0 = m0 + ar, r1 = m0 + 64 + ar;
    ra0 = r0 < T ? *reinterpret_cast<const float4*>(D + r0 * E + k0 + ak) : make_float4(0.f, 0.f, 0.f, 0.f);
    ra1 = r1 < T ? *reinterpret_cast<const float4*>(D + r1 * E + k0 + ak) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float* pb = C + (int64_t)(k0 + bk) * H + n0 + bn;
    rb0 = *reinterpret_cast<const float4*>(pb);
    rb1 = *reinterpret_cast<const float4*>(pb + 4);
  };
  auto store = [&]() {
    As[ak + 0][ar] = ra0.x; As[ak + 1][ar] = ra0.y; As[ak + 2][ar] = ra0.z; As[ak + 3][ar] = ra0.w;
    As[ak + 0][64 + ar] = ra1.x; As[ak + 1][64 + ar] = ra1.y;
    As[ak + 2][64 + ar] = ra1.z; As[ak + 3][64 + ar] = ra1.w;
    *reinterpret_cast<float4*>(&Bs[bk][bn]) = rb0;
    *reinterpret_cast<float4*>(&Bs[bk][bn + 4]) = rb1;
  };
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  load(0);
  for (int k0 = 0; k0 < E; k0 += DK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + DK < E) load(k0 + DK);
    tile_step(As, Bs, ty, tx, acc);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t t = m0 + 8 * ty + i;
    if (t >= T) break;
    const int64_t o = t * H + n0 + 8 * tx;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    if (dx_in) {
      const uint4 w = *reinterpret_cast<const uint4*>(dx_in + o);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_to_f32(ww[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_to_f32(ww[j] >> 16);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] += acc[i][j];
    *reinterpret_cast<uint4*>(dx_out + o) =
        make_uint4(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]),
                   f32x2_to_bf16x2(v[4], v[5]), f32x2_to_bf16x2(v[6], v[7]));
  }
}

// part[z][e, h] = sum over tokens t of slice z of dlogit[t, e] x[t, h]; grid
// (H / 128, ceil(E / 128), slices).  A = dlogit^T (read along e), B = x rows.
__global__ __launch_bounds__(DT) void dense_dc_kernel(
    const float* __restrict__ D, const uint16_t* __restrict__ x, int64_t T, int64_t H, int E,
    int64_t slice, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float As[DK][DP];
  __shared__ __attribute__((aligned(16))) float Bs[DK][DP];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t n0 = (int64_t)blockIdx.x * DN;
  const int m0 = blockIdx.y * DM;
  const int64_t t0 = (int64_t)blockIdx.z * slice, t1 = min(T, t0 + slice);
  // K row tid/16 of both tiles; A columns 8 (tid % 16) .. +7 (experts),
  // B columns 8 (tid % 16) .. +7 (hidden)
  const int kr = tid >> 4, c8 = (tid & 15) * 8;
  float4 ra0, ra1;
  uint4 rx;
  auto load = [&](int64_t k0) {
    const int64_t t = k0 + kr;
    const int e = m0 + c8;
    ra0 = make_float4(0.f, 0.f, 0.f, 0.f);
    ra1 = ra0;
    rx = make_uint4(0u, 0u, 0u, 0u);
    if (t < t1) {
      if (e < E) ra0 = *reinterpret_cast<const float4*>(D + t * E + e);
      if (e + 4 < E) ra1 = *reinterpret_cast<const float4*>(D + t * E + e + 4);
      rx = *reinterpret_cast<const uint4*>(x + t * H + n0 + c8);
    }
  };
  auto store = [&]() {
    *reinterpret_cast<float4*>(&As[kr][c8]) = ra0;
    *reinterpret_cast<float4*>(&As[kr][c8 + 4]) = ra1;
    const uint32_t ww[4] = {rx.x, rx.y, rx.z, rx.w};
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(ww[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_to_f32(ww[j] >> 16);
    }
    *reinterpret_cast<float4*>(&Bs[kr][c8]) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(&Bs[kr][c8 + 4]) = make_float4(v[4], v[5], v[6], v[7]);
  };
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  if (t0 < t1) load(t0);
  for (int64_t k0 = t0; k0 < t1; k0 += DK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + DK < t1) load(k0 + DK);
    tile_step(As, Bs, ty, tx, acc);
  }
  float* out = part + (int64_t)blockIdx.z * E * H;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = m0 + 8 * ty + i;
    if (e >= E) break;
    float* o = out + (int64_t)e * H + n0 + 8 * tx;
    *reinterpret_cast<float4*>(o) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
  }
}

__global__ __launch_bounds__(DT) void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * DT + threadIdx.x; i < n; i += (int64_t)gridDim.x * DT)
    p[i] = v;
}

// dC = sum over slices z = 0, 1, ... of part[z], in that order
__global__ __launch_bounds__(DT) void dc_reduce_kernel(const float* __restrict__ part,
                                                       int64_t n4, int slices,
                                                       float* __restrict__ dC) {
  for (int64_t i = (int64_t)blockIdx.x * DT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * DT) {
    float4 a = reinterpret_cast<const float4*>(part)[i];
    for (int z = 1; z < slices; ++z) {
      const float4 b = reinterpret_cast<const float4*>(part)[(int64_t)z * n4 + i];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    reinterpret_cast<float4*>(dC)[i] = a;
  }
}

// token slices of the centroid gradient: about 1024 tokens each (a multiple
// of the K step), at most 16
void dc_split(int64_t T, int64_t& slices, int64_t& slice) {
  slices = std::max<int64_t>(1, std::min<int64_t>(16, ceil_div(T, 1024)));
  slice = ceil_div(ceil_div(T, slices), DK) * DK;
  slices = ceil_div(T, slice);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_router_backward_dense_workspace_bytes(int64_t T, int64_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  int64_t slices, slice;
  dc_split(T, slices, slice);
  return slices > 1 ? (size_t)(slices * E * H) * sizeof(float) : 0;
}

extern "C" int moe_router_backward_dense(
    const void* x_bf16, const float* centroids, const int32_t* topk_idx, const float* d_topk_w,
    const float* scores, const float* score_sums, const float* seq_f, int64_t T, int64_t H,
    int32_t E, int32_t k, int64_t seq_len, float alpha, const void* dx_in_bf16, void* dx_out_bf16,
    float* d_centroids, float* dlogit, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && T < (1ll << 31), "moe_router_backward_dense: T=%lld out of range",
              (long long)T);
  MOE_INVALID(E >= 16 && E <= 256 && E % 16 == 0,
              "moe_router_backward_dense: E=%d must be a multiple of 16 in [16, 256]", (int)E);
  MOE_INVALID(k >= 1 && k <= 8, "moe_router_backward_dense: k=%d must be in [1, 8]", (int)k);
  MOE_INVALID(H > 0 && H % 128 == 0, "moe_router_backward_dense: H=%lld must be a positive multiple of 128",
              (long long)H);
  MOE_INVALID(seq_len >= 1 && seq_len <= 65536,
              "moe_router_backward_dense: seq_len=%lld must be in [1, 65536]", (long long)seq_len);
  MOE_INVALID(d_centroids, "moe_router_backward_dense: d_centroids is null");
  hipStream_t st = as_stream(stream);
  if (T == 0) {
    fill_f32_kernel<<<dim3(256), dim3(256), 0, st>>>(d_centroids, (int64_t)E * H, 0.0f);
    return check_launch("moe_router_backward_dense(fill)");
  }
  MOE_INVALID(x_bf16 && centroids && topk_idx && d_topk_w && scores && score_sums && seq_f &&
                  dx_out_bf16 && dlogit,
              "moe_router_backward_dense: null pointer");
  MOE_INVALID(dx_in_bf16 != dx_out_bf16, "moe_router_backward_dense: dx_in and dx_out alias");
  MOE_INVALID(((uintptr_t)x_bf16 & 15) == 0 && ((uintptr_t)centroids & 15) == 0 &&
                  ((uintptr_t)scores & 15) == 0 && ((uintptr_t)seq_f & 15) == 0 &&
                  ((uintptr_t)dx_in_bf16 & 15) == 0 && ((uintptr_t)dx_out_bf16 & 15) == 0 &&
                  ((uintptr_t)d_centroids & 15) == 0 && ((uintptr_t)dlogit & 15) == 0,
              "moe_router_backward_dense: x, centroids, scores, seq_f, dx_in, dx_out, d_centroids "
              "and dlogit must be 16-byte aligned");
  int64_t slices, slice;
  dc_split(T, slices, slice);
  const size_t need = moe_router_backward_dense_workspace_bytes(T, H, E);
  MOE_REQUIRE(need == 0 || (workspace != nullptr && workspace_bytes >= need &&
                            ((uintptr_t)workspace & 15) == 0),
              MOE_ERR_WORKSPACE,
              "moe_router_backward_dense: workspace needs %zu bytes (16-byte aligned), got %zu",
              need, workspace_bytes);
  MOE_UNSUPPORTED(ceil_div(T, DM) <= 65535, "moe_router_backward_dense: T too large");
  const uint16_t* x = static_cast<const uint16_t*>(x_bf16);
  dense_dlogit_kernel<<<dim3((unsigned)ceil_div(T, DT / 64)), dim3(DT), 0, st>>>(
      scores, score_sums, seq_f, topk_idx, d_topk_w, T, E, k, seq_len, alpha, dlogit);
  dense_dx_kernel<<<dim3((unsigned)(H / DN), (unsigned)ceil_div(T, DM)), dim3(DT), 0, st>>>(
      dlogit, centroids, static_cast<const uint16_t*>(dx_in_bf16), T, H, E,
      static_cast<uint16_t*>(dx_out_bf16));
  float* part = slices > 1 ? static_cast<float*>(workspace) : d_centroids;
  dense_dc_kernel<<<dim3((unsigned)(H / DN), (unsigned)ceil_div(E, DM), (unsigned)slices), dim3(DT),
                    0, st>>>(dlogit, x, T, H, E, slice, part);
  if (slices > 1) {
    const int64_t n4 = (int64_t)E * H / 4;
    dc_reduce_kernel<<<dim3((unsigned)std::min<int64_t>(ceil_div(n4, DT), 4096)), dim3(DT), 0, st>>>(
        part, n4, (int)slices, d_centroids);
  }
  return check_launch("moe_router_backward_dense");
}
