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
// Kernels:
//  1. router logits: l = x * C^T on bf16 MFMA.  x is bf16 (exact); each fp32
//     centroid is split exactly into three bf16 pieces (hi + mid + lo), so
//     every product is exact and only the fp32 accumulation rounds.  Small
//     batches (router_logits_kernel): a 64-token x 64-expert tile per
//     workgroup, partial sums kept per 512-wide K chunk; large batches
//     (router_logits_wide_kernel): the planes split once per call into the
//     workspace, 256 tokens x 256 experts per workgroup.  Either way the K
//     range may be split over workgroups; the partials are added in fixed
//     order by kernel 2.
//  2. router_select: one wave per token, 4 experts per lane (lane l owns
//     experts 4l..4l+3).  Group top-2 sums by merge rounds over the lanes of
//     a group, group ranks from each group's score read as a scalar, and the
//     top-k as a threshold on the biased scores' order-preserving bits built
//     from ballot counts (ties to the lower expert id).  The histogram is
//     built with LDS atomics and flushed with one global integer atomic per
//     expert and workgroup (integer adds: order-independent, so
//     deterministic).
//  3. bias_update: the +-gamma rule on the counts.
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

// ---- large batches: the centroids are split once per call into three bf16
// planes (hi, mid, lo; C = hi + mid + lo exactly) in the workspace, and a
// workgroup computes 256 tokens x 256 experts over a K range (split-K
// partials, added in fixed order by router_select) on
// v_mfma_f32_32x32x16_bf16: x is the row operand, each plane the column
// operand, all three into one accumulator.  Operands move global -> LDS by
// buffer_load ... lds copies into two 64 KB stages (x 256 rows x 64 B,
// planes 3 x 256 rows x 64 B); rows' 16 B chunks are XOR-swizzled so the
// operand reads are conflict-free.

constexpr int RW_TOK = 256;
constexpr int RW_XB = 256 * 64;            // x stage: 256 rows x 32 bf16
constexpr int RW_PB = 256 * 64;            // one plane's stage
constexpr int RW_STAGE = RW_XB + 3 * RW_PB;

typedef float v16f_r __attribute__((ext_vector_type(16)));
typedef int v4i_r __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int rw_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

__device__ __forceinline__ v4i_r rw_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4i_r r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Lane i's 16 bytes from buffer offset voff + soff land at m0 + IMM + i*16
// (soff moves the global address only; loads past the buffer return 0).
template <int IMM>
__device__ __forceinline__ void rw_copy(const v4i_r& r, uint32_t voff, uint32_t soff, uint32_t m0b) {
  asm volatile("s_add_u32 m0, %3, %4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(r), "s"(soff), "s"(m0b), "n"(IMM)
               : "memory", "m0", "scc");
}

__global__ void split_planes_kernel(const float* __restrict__ C, int64_t n,
                                    uint16_t* __restrict__ planes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t h, m, l;
    split3(C[i], h, m, l);
    planes[i] = (uint16_t)h;
    planes[n + i] = (uint16_t)m;
    planes[2 * n + i] = (uint16_t)l;
  }
}

__global__ __launch_bounds__(512, 1) void router_logits_wide_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, const uint16_t* __restrict__ planes,
    int E, int64_t kper, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * RW_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;  // tokens 64wm.., experts 128wn..
  const int q = lane >> 5, l32 = lane & 31;
  const int64_t tok0 = (int64_t)blockIdx.x * RW_TOK;
  const int64_t k0 = (int64_t)blockIdx.y * kper;
  const int nst = (int)((min<int64_t>(H, k0 + kper) - k0) >> 5);  // 32-K steps
  const uint32_t rowb = (uint32_t)H * 2;

  // copies: waves 0, 1 move x rows 128(wv&1).., waves 2..7 plane (wv-2)/2's
  // expert rows 128(wv&1)..; copy c (0..7) covers 16 rows: lane -> row
  // +lane/4, LDS slot lane%4 <- global chunk (lane%4) ^ rw_swz(row)
  const int rl = 128 * (wv & 1) + (lane >> 2);
  const uint32_t gch = (uint32_t)((lane & 3) ^ rw_swz(rl));
  v4i_r rs;
  uint32_t voff;
  uint32_t region;
  if (wv < 2) {
    rs = rw_rsrc(x, (uint32_t)T * rowb);
    voff = (uint32_t)(tok0 + rl) * rowb + gch * 16;
    region = 0;
  } else {
    const int pl = (wv - 2) >> 1;
    rs = rw_rsrc(planes, 3u * (uint32_t)E * rowb);
    voff = (uint32_t)(pl * E + rl) * rowb + gch * 16;
    region = RW_XB + pl * RW_PB;
  }
  const uint32_t m0b = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)smem + region + (uint32_t)(128 * (wv & 1)) * 64));
  const uint32_t s16 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(16 * rowb));
  auto copy_step = [&](auto ST_, int st) __attribute__((always_inline)) {
    constexpr int ST = decltype(ST_)::value;
    const uint32_t so = (uint32_t)(k0 + 32 * st) * 2;
    rw_copy<ST * RW_STAGE + 0 * 1024>(rs, voff, so, m0b);
    rw_copy<ST * RW_STAGE + 1 * 1024>(rs, voff, so + s16, m0b);
    rw_copy<ST * RW_STAGE + 2 * 1024>(rs, voff, so + 2 * s16, m0b);
    rw_copy<ST * RW_STAGE + 3 * 1024>(rs, voff, so + 3 * s16, m0b);
    rw_copy<ST * RW_STAGE + 4 * 1024>(rs, voff, so + 4 * s16, m0b);
    rw_copy<ST * RW_STAGE + 5 * 1024>(rs, voff, so + 5 * s16, m0b);
    rw_copy<ST * RW_STAGE + 6 * 1024>(rs, voff, so + 6 * s16, m0b);
    rw_copy<ST * RW_STAGE + 7 * 1024>(rs, voff, so + 7 * s16, m0b);
  };

  v16f_r acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // operand reads: lane's 16 B (K 8q..8q+7 of half kh) of row l32 + 32i
  const int sw = rw_swz(l32);
  const uint8_t* pa[2];
  const uint8_t* pb[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int o = l32 * 64 + (((2 * kh + q) ^ sw) << 4);
    pa[kh] = smem + wm * 64 * 64 + o;
    pb[kh] = smem + RW_XB + wn * 128 * 64 + o;
  }
  auto compute = [&](auto ST_) __attribute__((always_inline)) {
    constexpr int ST = decltype(ST_)::value;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      v8bf a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const v8bf*>(pa[kh] + ST * RW_STAGE + i * 32 * 64);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8bf b = *reinterpret_cast<const v8bf*>(pb[kh] + ST * RW_STAGE + pl * RW_PB + j * 32 * 64);
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i][j], 0, 0, 0);
        }
    }
  };

  copy_step(std::integral_constant<int, 0>(), 0);
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) copy_step(std::integral_constant<int, 1>(), st + 1);
    compute(std::integral_constant<int, 0>());
    __builtin_amdgcn_s_waitcnt(7 << 4);
    __builtin_amdgcn_s_barrier();
    if (st + 1 < nst) {
      if (st + 2 < nst) copy_step(std::integral_constant<int, 0>(), st + 2);
      compute(std::integral_constant<int, 1>());
      __builtin_amdgcn_s_waitcnt(7 << 4);
      __builtin_amdgcn_s_barrier();
    }
  }

  // result element r of lane l: token 8(r/4) + 4q + r%4 of row block i,
  // expert l32 of block j
  float* out = part + (int64_t)blockIdx.y * T * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 128 * wn + 32 * j + l32;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = tok0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
        if (t < T && e < E) out[t * E + e] = acc[i][j][r];
      }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// The value of the lane paired with this one in the merge round of width o
// (o = 1, 2, 4, 8): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror.
__device__ __forceinline__ float dpp_pair(float v, int o) {
  const int x = __float_as_int(v);
  int r;
  switch (o) {
    case 1: r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}

template <bool PF>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int KS, int64_t T, const float* __restrict__ bias, int E,
    int n_group, int topk_group, int k, int lpg, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ counts, float* __restrict__ scores,
    float* __restrict__ score_sums,
    float* __restrict__ topk_s) {
  __shared__ int hist[256];
  __shared__ int s_sel_e[4][8];    // per wave: the token's selection in expert order
  __shared__ float s_sel_s[4][8];
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

  // PF (at most 8 split-K partials): a wave requests its next token's
  // partials before the current token's selection runs, so their memory
  // round trip overlaps it; otherwise eight splits at a time are requested
  // before the first of them is added.  Either way they are added in split
  // order.
  const int64_t tstride = (int64_t)gridDim.x * 4;
  float4 nx[8];
  const int64_t kstride = T * E;  // between split-K partials
  auto fetch = [&](int64_t tt) {
    if (tt < T && active) {
      const float* p = part + tt * E + ebase;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < KS) nx[u] = *reinterpret_cast<const float4*>(p + u * kstride);
    }
  };
  if (PF) fetch((int64_t)blockIdx.x * 4 + wv);
  for (int64_t t = (int64_t)blockIdx.x * 4 + wv; t < T; t += tstride) {
    float lg[4] = {0.f, 0.f, 0.f, 0.f};
    if (PF) {
      if (active) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (u < KS) {
            lg[0] += nx[u].x;
            lg[1] += nx[u].y;
            lg[2] += nx[u].z;
            lg[3] += nx[u].w;
          }
      }
      fetch(t + tstride);
    } else if (active) {
      for (int k0 = 0; k0 < KS; k0 += 8) {
        float4 pv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (k0 + u < KS)
            pv[u] = *reinterpret_cast<const float4*>(part + ((int64_t)(k0 + u) * T + t) * E + ebase);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (k0 + u < KS) {
            lg[0] += pv[u].x;
            lg[1] += pv[u].y;
            lg[2] += pv[u].z;
            lg[3] += pv[u].w;
          }
      }
    }
    float s[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = 1.0f / (1.0f + expf(-lg[i]));
      sb[i] = active ? s[i] + b[i] : -INFINITY;
    }
    if (scores) {  // every routed expert's unbiased score, and their sum
      float ls = 0.f;
      if (active) {
        *reinterpret_cast<float4*>(scores + t * E + ebase) = make_float4(s[0], s[1], s[2], s[3]);
        ls = (s[0] + s[1]) + (s[2] + s[3]);
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) ls += __shfl_xor(ls, o, 64);
      if (lane == 0) score_sums[t] = ls;
    }
    // top-2 of this lane's 4 biased scores, then of the group's lanes
    float t1 = fmaxf(sb[0], sb[1]), t2 = fminf(sb[0], sb[1]);
#pragma unroll
    for (int i = 2; i < 4; ++i) {
      const float v = sb[i];
      t2 = fmaxf(t2, fminf(t1, v));
      t1 = fmaxf(t1, v);
    }
    // merge rounds pair each lane with one holding the top-2 of a disjoint
    // set of the group's lanes: xor 1 and xor 2 within a quad, then the
    // mirror lane in a half row (i <-> 7 - i) and in a row (i <-> 15 - i),
    // all lane moves within the row (DPP); wider groups exchange by xor
    for (int o = 1; o < lpg; o <<= 1) {
      float o1, o2;
      if (o <= 8) {
        o1 = dpp_pair(t1, o);
        o2 = dpp_pair(t2, o);
      } else {
        o1 = __shfl_xor(t1, o, 64);
        o2 = __shfl_xor(t2, o, 64);
      }
      t2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
      t1 = fmaxf(t1, o1);
    }
    const float gscore = t1 + t2;
    // group j's score sits in lane j * lpg (read as a scalar)
    int rank = 0;
    for (int j = 0; j < n_group; ++j) {
      const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gscore), j * lpg));
      rank += (sj > gscore || (sj == gscore && j < gid)) ? 1 : 0;
    }
    const bool kept = active && rank < topk_group;
    // top-k among the kept experts, in the order (biased score descending,
    // expert id ascending).  Each slot's key is the order-preserving bits
    // of its biased score (-0 as +0), 0 for slots outside the kept groups
    // (below every kept one).  A threshold is built bit by bit from the top:
    // a bit stays set when at least k keys reach the prefix with it (counted
    // by ballots), so the keys at or above the prefix always include the k
    // largest; as soon as exactly k keys reach it they are the selection and
    // the search stops.  Otherwise it ends on the k-th largest key itself,
    // shared by several slots: every slot above it is taken, and of those
    // equal to it the ones with the lowest expert ids, as many as are left.
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = sb[i] == 0.0f ? 0u : __float_as_uint(sb[i]);  // -0 ties +0
      const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key[i] = kept ? ord : 0u;
    }
    // every kept key shares the bits above the highest bit where the largest
    // and the smallest kept key differ: the search would set exactly those
    // (at least k keys reach each of them, no key reaches a zero one), so it
    // starts below them
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kmax = max(kmax, key[i]);
      if (kept) kmin = min(kmin, key[i]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    }
    const uint32_t diff = kmax ^ kmin;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;  // highest differing bit
    uint32_t pre = top < 0 ? kmax : top >= 31 ? 0u : kmax & ~((2u << top) - 1u);
    bool exact = false;
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t c = pre | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(key[i] >= c));
      if (cnt >= k) {
        pre = c;
        if (cnt == k) {
          exact = true;
          break;
        }
      }
    }
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    uint64_t msk[4];
    if (exact) {
#pragma unroll
      for (int i = 0; i < 4; ++i) msk[i] = __ballot(key[i] >= pre);
    } else {
      // slots equal to the k-th key, ranked by expert id (e = 4 lane + i):
      // equal slots of the lanes below, then this lane's earlier ones
      uint64_t eq[4];
      int left = k, tie = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        msk[i] = __ballot(key[i] > pre);
        eq[i] = __ballot(key[i] == pre);
        left -= __popcll(msk[i]);
        tie += __popcll(eq[i] & lanes_below);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool mine = (eq[i] >> lane) & 1ull;
        msk[i] |= __ballot(mine && tie < left);
        tie += mine ? 1 : 0;
      }
    }
    // ranks in ascending expert id (e = 4 lane + i): selected slots of the
    // lanes below, then this lane's earlier slots; each selected slot puts
    // (e, s) at its rank, and the wave reads the k entries back in order
    int below = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) below += __popcll(msk[i] & lanes_below);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((msk[i] >> lane) & 1ull) {
        s_sel_e[wv][below] = ebase + i;
        s_sel_s[wv][below] = s[i];
        ++below;
      }
    }
    float sum = 0.f;
    int my_e = 0;
    float my_s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const float sj = s_sel_s[wv][j];
        sum += sj;
        if (j == lane) {
          my_e = s_sel_e[wv][j];
          my_s = sj;
        }
      }
    }
    my_e = min(my_e, E - 1);  // only reachable with NaN scores (unspecified input)
    if (lane < k) {
      topk_idx[t * k + lane] = my_e;
      topk_w[t * k + lane] = my_s / sum;
      if (topk_s) topk_s[t * k + lane] = my_s;
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
  bool wide;  // the 256-token kernel with pre-split planes
};

// the 256-token kernel: large batches whose x and planes fit 32-bit offsets
bool route_wide(int64_t T, int64_t H, int32_t E) {
  return T >= 2048 && E <= 256 && H % 256 == 0 && T * H * 2 < ((int64_t)1 << 32) &&
         3 * (int64_t)E * H * 2 < ((int64_t)1 << 32);
}

RouteSplit route_split(int64_t T, int64_t H, int32_t E) {
  if (route_wide(T, H, E)) {
    const int64_t tiles = ceil_div(T, RW_TOK);
    int64_t ks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(256, tiles), H / 256));
    const int64_t kper = ceil_div(ceil_div(H, ks), 32) * 32;
    ks = ceil_div(H, kper);
    return {ks, kper, true};
  }
  const int64_t tiles = ceil_div(T, RT_TOK) * ceil_div(E, RT_EXP);
  int64_t ks = std::max<int64_t>(1, ceil_div(1024, std::max<int64_t>(tiles, 1)));
  ks = std::min<int64_t>(std::min<int64_t>(ks, 1024), std::max<int64_t>(1, H / 256));
  int64_t kper = ceil_div(ceil_div(H, ks), RT_KC) * RT_KC;
  ks = ceil_div(H, kper);
  return {ks, kper, false};
}

// workspace: the split-K partials [ks, T, E] fp32, then (wide) the planes
size_t route_ws_partials(const RouteSplit& sp, int64_t T, int32_t E) {
  return ((size_t)(sp.ks * T * E) * sizeof(float) + 255) / 256 * 256;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_route_workspace_bytes(int64_t T, int64_t H, int32_t E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  const RouteSplit sp = route_split(T, H, E);
  return route_ws_partials(sp, T, E) + (sp.wide ? (size_t)3 * E * H * sizeof(uint16_t) : 0);
}

namespace {

int route_impl(const void* x_bf16, int64_t T, int64_t H, const float* centroids,
               const float* bias, int32_t E, int32_t n_group, int32_t topk_group, int32_t k,
               int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* workspace,
               size_t workspace_bytes, float* scores, float* score_sums, float* topk_s,
               void* stream) {
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
  MOE_INVALID(((uintptr_t)topk_s & 3) == 0, "moe_route: topk_s must be 4-byte aligned");
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
  if (sp.wide) {
    uint16_t* planes = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) +
                                                   route_ws_partials(sp, T, E));
    split_planes_kernel<<<dim3(1024), dim3(256), 0, st>>>(centroids, (int64_t)E * H, planes);
    router_logits_wide_kernel<<<dim3((unsigned)ceil_div(T, RW_TOK), (unsigned)sp.ks), dim3(512), 0,
                                st>>>(static_cast<const uint16_t*>(x_bf16), T, H, planes, E,
                                      sp.kper, part);
  } else {
    router_logits_kernel<<<dim3((unsigned)ceil_div(T, RT_TOK), (unsigned)ceil_div(E, RT_EXP),
                                (unsigned)sp.ks),
                           dim3(256), 0, st>>>(static_cast<const uint16_t*>(x_bf16), T, H,
                                               centroids, E, sp.kper, part);
  }
  // four tokens per workgroup per round; 1024 workgroups (four per CU at
  // 96 VGPRs: one round of residency) give a prefetching wave several tokens
  const int64_t sel_blocks = std::min<int64_t>(ceil_div(T, 4), 1024);
  if (sp.ks <= 8)
    router_select_kernel<true><<<dim3((unsigned)sel_blocks), dim3(256), 0, st>>>(
        part, (int)sp.ks, T, bias, E, n_group, topk_group, k, lpg, topk_idx, topk_w,
        expert_counts, scores, score_sums, topk_s);
  else
    router_select_kernel<false><<<dim3((unsigned)sel_blocks), dim3(256), 0, st>>>(
        part, (int)sp.ks, T, bias, E, n_group, topk_group, k, lpg, topk_idx, topk_w,
        expert_counts, scores, score_sums, topk_s);
  return check_launch("moe_route");
}

}  // namespace

extern "C" int moe_route(const void* x_bf16, int64_t T, int64_t H, const float* centroids,
                         const float* bias, int32_t E, int32_t n_group, int32_t topk_group,
                         int32_t k, int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                         void* workspace, size_t workspace_bytes, float* topk_s, void* stream) {
  clear_error();
  return route_impl(x_bf16, T, H, centroids, bias, E, n_group, topk_group, k, topk_idx, topk_w,
                    expert_counts, workspace, workspace_bytes, nullptr, nullptr, topk_s, stream);
}

extern "C" int moe_route_scores(const void* x_bf16, int64_t T, int64_t H,
                                const float* centroids, const float* bias, int32_t E,
                                int32_t n_group, int32_t topk_group, int32_t k,
                                int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                                void* workspace, size_t workspace_bytes, float* scores,
                                float* score_sums, float* topk_s, void* stream) {
  clear_error();
  MOE_INVALID(T == 0 || (scores && score_sums), "moe_route_scores: scores or score_sums is null");
  MOE_INVALID(((uintptr_t)scores & 15) == 0, "moe_route_scores: scores must be 16-byte aligned");
  return route_impl(x_bf16, T, H, centroids, bias, E, n_group, topk_group, k, topk_idx, topk_w,
                    expert_counts, workspace, workspace_bytes, scores, score_sums, topk_s, stream);
}

extern "C" int moe_bias_update(const int32_t* expert_counts, float* bias, int32_t E, float gamma,
                               void* stream) {
  clear_error();
  MOE_INVALID(E >= 1 && E <= 1024, "moe_bias_update: E=%d must be in [1, 1024]", (int)E);
  MOE_INVALID(expert_counts && bias, "moe_bias_update: null pointer");
  bias_update_kernel<<<1, 256, 0, as_stream(stream)>>>(expert_counts, bias, E, gamma);
  return check_launch("moe_bias_update");
}
