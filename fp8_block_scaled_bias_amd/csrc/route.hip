// Router (sigmoid gate, selection bias, group-limited top-k, expert-count
// histogram) and the aux-loss-free bias update.
//
// Method: aliyun study note (developer.aliyun.com/article/1776647) section
// 2.2 - a sigmoid score per expert and a per-expert bias that only moves the
// choice, raised for underloaded and lowered for overloaded experts;
// news.qq.com/rain/a/20241229A05OQF00, sections DeepSeekMoE 架构 (8 of 256
// routed experts per token), 节点限制路由 (at most 4 nodes per token) and
// 无额外损耗的负载均衡 (bias update speed 0.001).
//
// Two kernels:
//  1. router_logits: l = x * C^T on bf16 MFMA.  x is bf16 (exact); each fp32
//     centroid is split exactly into three bf16 pieces (hi + mid + lo), so
//     every product is exact and only the fp32 accumulation rounds.  Partial
//     sums are kept per 512-wide K chunk and then added, which keeps the
//     accumulator's rounding error near that of a short fp32 sum.  A 64-token
//     x 64-expert tile per workgroup; for small T the K range is split over
//     workgroups and the partials are added in fixed order by kernel 2.
//  2. router_select: one wave per token, 4 experts per lane (lane l owns
//     experts 4l..4l+3).  Group top-2 sums are butterflies over the lanes of a
//     group, group ranks are counted over shuffled group scores, and the k
//     winners are k wave-wide argmax rounds.  The histogram is built with LDS
//     atomics and flushed with one global integer atomic per expert and
//     workgroup (integer adds: order-independent, so deterministic).
#include "common.h"

namespace moe {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int RT_TOK = 64;   // tokens per workgroup
constexpr int RT_EXP = 64;   // experts per workgroup
constexpr int RT_KC = 64;    // K elements per LDS stage
constexpr int RT_PAD = 8;    // bf16 padding per LDS row (row = 144 B: no bank conflicts)
constexpr int RT_CHUNK = 8;  // stages per accumulation chunk (512 K)

__device__ __forceinline__ void split3(float c, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t u = __float_as_uint(c);
  hi = u >> 16;
  const float r1 = c - __uint_as_float(u & 0xFFFF0000u);  // exact
  const uint32_t u1 = __float_as_uint(r1);
  mid = u1 >> 16;
  const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);  // exact, <= 8 significant bits
  lo = __float_as_uint(r2) >> 16;                           // exact truncation
}

__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, const float* __restrict__ C, int E,
    int64_t kper, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[RT_TOK][RT_KC + RT_PAD];
  __shared__ __attribute__((aligned(16))) uint16_t cs[3][RT_EXP][RT_KC + RT_PAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int64_t tok0 = (int64_t)blockIdx.x * RT_TOK;
  const int e0 = blockIdx.y * RT_EXP;
  const int64_t k0 = (int64_t)blockIdx.z * kper;
  const int64_t k1 = std::min<int64_t>(H, k0 + kper);

  v4f acc[4], tmp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    tmp[j] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  int stage = 0;
  for (int64_t kc = k0; kc < k1; kc += RT_KC, ++stage) {
    // x tile: 64 rows x 128 B = 512 x 16 B
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      const int row = c >> 3, col = (c & 7) * 8;
      const int64_t t = tok0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < T) v = *reinterpret_cast<const uint4*>(x + t * H + kc + col);
      *reinterpret_cast<uint4*>(&xs[row][col]) = v;
    }
    // centroid tile: 64 experts x 64 fp32 = 1024 x 16 B, split into 3 bf16 planes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int er = c >> 4, col = (c & 15) * 4;
      const int e = e0 + er;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E) v = *reinterpret_cast<const float4*>(C + (int64_t)e * H + kc + col);
      uint32_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
      split3(v.x, h0, m0, l0);
      split3(v.y, h1, m1, l1);
      split3(v.z, h2, m2, l2);
      split3(v.w, h3, m3, l3);
      *reinterpret_cast<uint2*>(&cs[0][er][col]) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      *reinterpret_cast<uint2*>(&cs[1][er][col]) = make_uint2(m0 | (m1 << 16), m2 | (m3 << 16));
      *reinterpret_cast<uint2*>(&cs[2][er][col]) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < RT_KC / 32; ++ks) {
      const int kk = ks * 32 + 8 * (lane >> 4);
      const v8bf a = *reinterpret_cast<const v8bf*>(&xs[wv * 16 + (lane & 15)][kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const v8bf b = *reinterpret_cast<const v8bf*>(&cs[p][j * 16 + (lane & 15)][kk]);
          tmp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, tmp[j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if ((stage + 1) % RT_CHUNK == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[j] += tmp[j];
        tmp[j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] += tmp[j];

  // D layout of 16x16 MFMA: lane holds rows 4*(lane/16)+r, column lane%16
  float* out = part + (int64_t)blockIdx.z * T * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + j * 16 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = tok0 + wv * 16 + 4 * (lane >> 4) + r;
      if (t < T && e < E) out[t * E + e] = acc[j][r];
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__device__ __forceinline__ bool beats(float v, int e, float ov, int oe) {
  return ov > v || (ov == v && oe < e);
}

__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int KS, int64_t T, const float* __restrict__ bias, int E,
    int n_group, int topk_group, int k, int lpg, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ counts) {
  __shared__ int hist[256];
  for (int i = threadIdx.x; i < 256; i += 256) hist[i] = 0;
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ebase = lane * 4;
  const bool active = ebase < E;
  const int gid = active ? lane / lpg : n_group;
  float b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = active ? bias[ebase + i] : 0.f;

  for (int64_t t = (int64_t)blockIdx.x * 4 + wv; t < T; t += (int64_t)gridDim.x * 4) {
    float lg[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      for (int ks = 0; ks < KS; ++ks) {
        const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)ks * T + t) * E + ebase);
        lg[0] += v.x;
        lg[1] += v.y;
        lg[2] += v.z;
        lg[3] += v.w;
      }
    }
    float s[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = 1.0f / (1.0f + expf(-lg[i]));
      sb[i] = active ? s[i] + b[i] : -INFINITY;
    }
    // top-2 of this lane's 4 biased scores, then of the group's lanes
    float t1 = fmaxf(sb[0], sb[1]), t2 = fminf(sb[0], sb[1]);
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      const float v = sb[i];
      t2 = fmaxf(t2, fminf(t1, v));
      t1 = fmaxf(t1, v);
    }
    for (int o = 1; o < lpg; o <<= 1) {
      const float o1 = __shfl_xor(t1, o, 64);
      const float o2 = __shfl_xor(t2, o, 64);
      t2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
      t1 = fmaxf(t1, o1);
    }
    const float gscore = t1 + t2;
    int rank = 0;
    for (int j = 0; j < n_group; ++j) {
      const float sj = __shfl(gscore, j * lpg, 64);
      rank += (sj > gscore || (sj == gscore && j < gid)) ? 1 : 0;
    }
    const bool kept = active && rank < topk_group;
    float cand[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cand[i] = kept ? sb[i] : -INFINITY;

    int sel[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      if (it < k) {
        float bv = cand[0];
        int be = ebase;
#pragma unroll
        for (int i = 1; i < 4; ++i)
          if (cand[i] > bv) {
            bv = cand[i];
            be = ebase + i;
          }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int oe = __shfl_xor(be, o, 64);
          if (beats(bv, be, ov, oe)) {
            bv = ov;
            be = oe;
          }
        }
        sel[it] = be;
        if ((be >> 2) == lane) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((be & 3) == i) cand[i] = -INFINITY;
        }
      } else {
        sel[it] = 0x7FFFFFFF;
      }
    }
    // ascending expert id (uniform across the wave)
#pragma unroll
    for (int i = 1; i < 8; ++i) {
#pragma unroll
      for (int j = i; j > 0; --j) {
        if (sel[j] < sel[j - 1]) {
          const int tmp = sel[j];
          sel[j] = sel[j - 1];
          sel[j - 1] = tmp;
        }
      }
    }
    float sv[8];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const int e = sel[j];
        float mine = s[0];
#pragma unroll
        for (int i = 1; i < 4; ++i)
          if ((e & 3) == i) mine = s[i];
        sv[j] = __shfl(mine, e >> 2, 64);
        sum += sv[j];
      } else {
        sv[j] = 0.f;
      }
    }
    int my_e = 0;
    float my_s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j == lane) {
        my_e = sel[j];
        my_s = sv[j];
      }
    my_e = min(my_e, E - 1);  // only reachable with NaN scores (unspecified input)
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = my_s / sum;
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    const int c = hist[e];
    if (c) atomicAdd(&counts[e], c);
  }
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts,
                                                          float* __restrict__ bias, int E,
                                                          float gamma) {
  __shared__ long long red[4];
  long long s = 0;
  for (int e = threadIdx.x; e < E; e += 256) s += counts[e];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  const long long total = red[0] + red[1] + red[2] + red[3];
  for (int e = threadIdx.x; e < E; e += 256) {
    const long long ce = (long long)counts[e] * E;
    const float b = bias[e];
    if (ce > total)
      bias[e] = b - gamma;
    else if (ce < total)
      bias[e] = b + gamma;
  }
}

struct RouteSplit {
  int64_t ks, kper;
};

RouteSplit route_split(int64_t T, int64_t H, int32_t E) {
  const int64_t tiles = ceil_div(T, RT_TOK) * ceil_div(E, RT_EXP);
  int64_t ks = std::max<int64_t>(1, ceil_div(1024, std::max<int64_t>(tiles, 1)));
  ks = std::min<int64_t>(std::min<int64_t>(ks, 1024), std::max<int64_t>(1, H / 256));
  int64_t kper = ceil_div(ceil_div(H, ks), RT_KC) * RT_KC;
  ks = ceil_div(H, kper);
  return {ks, kper};
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_workspace_bytes(int64_t T, int64_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  const RouteSplit sp = route_split(T, H, E);
  return (size_t)(sp.ks * T * E) * sizeof(float);
}

extern "C" int moe_route(const void* x_bf16, int64_t T, int64_t H, const float* centroids,
                         const float* bias, int32_t E, int32_t n_group, int32_t topk_group,
                         int32_t k, int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                         void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0, "moe_route: T=%lld < 0", (long long)T);
  MOE_INVALID(H > 0 && H % 128 == 0, "moe_route: H=%lld must be a positive multiple of 128",
              (long long)H);
  MOE_INVALID(E >= 2, "moe_route: E=%d < 2", (int)E);
  MOE_INVALID(n_group >= 1 && E % n_group == 0, "moe_route: E=%d not divisible by n_group=%d",
              (int)E, (int)n_group);
  MOE_INVALID(topk_group >= 1 && topk_group <= n_group,
              "moe_route: topk_group=%d must be in [1, n_group=%d]", (int)topk_group, (int)n_group);
  const int gsz = E / n_group;
  MOE_INVALID(gsz >= 2, "moe_route: group size %d < 2 (group score is a top-2 sum)", gsz);
  MOE_INVALID(k >= 1 && k <= topk_group * gsz, "moe_route: k=%d must be in [1, %d]", (int)k,
              topk_group * gsz);
  MOE_UNSUPPORTED(E <= 256, "moe_route: E=%d > 256 experts is not supported", (int)E);
  MOE_UNSUPPORTED(k <= 8, "moe_route: k=%d > 8 is not supported", (int)k);
  MOE_UNSUPPORTED(gsz % 4 == 0 && ((gsz / 4) & (gsz / 4 - 1)) == 0,
                  "moe_route: group size %d must be 4 times a power of two", gsz);
  MOE_INVALID(expert_counts, "moe_route: expert_counts is null");
  const int lpg = gsz / 4;
  hipStream_t st = as_stream(stream);
  if (T == 0) {
    fill_i32_kernel<<<1, 256, 0, st>>>(expert_counts, E, 0);
    return check_launch("moe_route(fill)");
  }
  MOE_INVALID(x_bf16 && centroids && bias && topk_idx && topk_w, "moe_route: null pointer");
  MOE_INVALID(((uintptr_t)x_bf16 & 15) == 0 && ((uintptr_t)centroids & 15) == 0,
              "moe_route: x and centroids must be 16-byte aligned");
  const size_t need = moe_route_workspace_bytes(T, H, E);
  MOE_REQUIRE(workspace != nullptr && workspace_bytes >= need && ((uintptr_t)workspace & 15) == 0,
              MOE_ERR_WORKSPACE, "moe_route: workspace needs %zu bytes (16-byte aligned), got %zu",
              need, workspace_bytes);
  MOE_UNSUPPORTED(ceil_div(T, RT_TOK) <= 0x7FFFFFFF, "moe_route: T too large");
  const RouteSplit sp = route_split(T, H, E);
  float* part = static_cast<float*>(workspace);

  fill_i32_kernel<<<1, 256, 0, st>>>(expert_counts, E, 0);
  router_logits_kernel<<<dim3((unsigned)ceil_div(T, RT_TOK), (unsigned)ceil_div(E, RT_EXP),
                              (unsigned)sp.ks),
                         dim3(256), 0, st>>>(static_cast<const uint16_t*>(x_bf16), T, H,
                                             centroids, E, sp.kper, part);
  const int64_t sel_blocks = std::min<int64_t>(ceil_div(T, 4), 2048);
  router_select_kernel<<<dim3((unsigned)sel_blocks), dim3(256), 0, st>>>(
      part, (int)sp.ks, T, bias, E, n_group, topk_group, k, lpg, topk_idx, topk_w,
      expert_counts);
  return check_launch("moe_route");
}

extern "C" int moe_bias_update(const int32_t* expert_counts, float* bias, int32_t E, float gamma,
                               void* stream) {
  clear_error();
  MOE_INVALID(E >= 1 && E <= 1024, "moe_bias_update: E=%d must be in [1, 1024]", (int)E);
  MOE_INVALID(expert_counts && bias, "moe_bias_update: null pointer");
  bias_update_kernel<<<1, 256, 0, as_stream(stream)>>>(expert_counts, bias, E, gamma);
  return check_launch("moe_bias_update");
}
