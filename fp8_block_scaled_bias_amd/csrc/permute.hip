// Dispatch: stable expert-major permutation of the token-expert assignments
// (the all-to-all dispatch step of a DualPipe chunk, news.qq.com/rain/a/
// 20241229A05OQF00 section DualPipe 流水线并行, done inside one GPU).
//
// Three passes, all integer work (bit-exact, deterministic):
//  1. permute_count   - one wave per 64-token chunk: per-chunk histogram.
//  2. permute_scan    - one workgroup per expert: exclusive scan of that
//                       expert's chunk counts, offset by the expert's start
//                       (sum of the counts of lower experts).
//  3. permute_scatter - one wave per chunk walks its assignments in
//                       (token, slot) order, 64 at a time; lanes holding the
//                       same expert find each other with 64-bit ballots over
//                       the id bits, take rank = popcount(lower matching
//                       lanes), and the last of them advances the expert's
//                       running position in LDS.  So rows of an expert come
//                       out in ascending (token, slot) order.
// An optional gather copies the E4M3 rows and 1x128 scales into row order.
#include "common.h"

#include <mutex>

namespace moe {
namespace {

constexpr int PM_TOK = 64;  // tokens per chunk

// Scratch of moe_permute_noalloc: one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// names a stand-in, not device memory); it uses the per-device address that
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) uint8_t scratch[MOE_PERMUTE_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of this device's scratch (NULL with the error set on failure).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("moe_permute_noalloc: no current device (or device id %d out of range)", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("moe_permute_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

__global__ __launch_bounds__(64) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                           int64_t T, int k, int E,
                                                           int32_t* __restrict__ hist) {
  extern __shared__ int h[];
  const int lane = threadIdx.x;
  const int64_t chunk = blockIdx.x;
  for (int e = lane; e < E; e += 64) h[e] = 0;
  __syncthreads();
  const int64_t t0 = chunk * PM_TOK;
  const int n = PM_TOK * k;
  for (int a = lane; a < n; a += 64) {
    const int64_t t = t0 + a / k;
    if (t < T) atomicAdd(&h[idx[t * k + a % k]], 1);
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) hist[chunk * E + e] = h[e];
}

// Block-wide (256 threads) inclusive scan of one value per thread.
__device__ __forceinline__ int block_inclusive_scan(int v, int* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  if (lane == 63) red[wv] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wv; ++w) add += red[w];
  const int res = v + add;
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(256) void permute_scan_kernel(const int32_t* __restrict__ counts,
                                                           int E, int64_t T, int k, int n_shared,
                                                           int64_t NB, int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int red[4];
  __shared__ int carry_s;
  const int e = blockIdx.x;
  // start of expert e: sum of counts of lower experts
  int part = 0;
  for (int i = threadIdx.x; i < e; i += 256) part += counts[i];
  const int lane = threadIdx.x & 63;
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (lane == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  const int start = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  if (threadIdx.x == 0) {
    offsets[e] = start;
    carry_s = start;
  }
  if (e == E - 1 && threadIdx.x == 0) {
    const int32_t routed = start + counts[e];
    for (int s = 0; s <= n_shared; ++s) offsets[E + s] = routed + (int32_t)(s * T);
  }
  __syncthreads();
  for (int64_t b0 = 0; b0 < NB; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const int v = b < NB ? hist[b * E + e] : 0;
    const int inc = block_inclusive_scan(v, red);
    const int carry = carry_s;
    if (b < NB) hist[b * E + e] = carry + inc - v;
    __syncthreads();
    if (threadIdx.x == 255) carry_s = carry + inc;
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int k, int E, int nbits,
    const int32_t* __restrict__ base, int n_shared, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ inv_perm) {
  extern __shared__ int run[];
  const int lane = threadIdx.x;
  const int64_t chunk = blockIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = base[chunk * E + e];
  run[E] = 0;  // sentinel bin for padding lanes (E + 1 ints allocated)
  __syncthreads();
  const int64_t t0 = chunk * PM_TOK;
  const int n = PM_TOK * k;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int a0 = 0; a0 < n; a0 += 64) {
    const int a = a0 + lane;
    const int64_t t = t0 + a / k;
    const bool valid = a < n && t < T;
    const int e = valid ? idx[t * k + a % k] : E;
    uint64_t m = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bal = __ballot(on);
      m &= on ? bal : ~bal;
    }
    const int rank = __popcll(m & lt);
    const int pos = run[e] + rank;
    __builtin_amdgcn_wave_barrier();
    const int last = 63 - __clzll(m);
    if (lane == last) run[e] = pos + 1;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      perm_src[pos] = (int32_t)t;
      inv_perm[t * k + a % k] = pos;
    }
    __syncthreads();
  }
  for (int s = 0; s < n_shared; ++s) {
    const int64_t t = t0 + lane;
    if (lane < PM_TOK && t < T) perm_src[T * k + s * T + t] = (int32_t)t;
  }
}

// a_out[r] = xq[perm_src[r]] (H bytes), a_scale_out[r] = xs[perm_src[r]] (H/128 floats)
__global__ __launch_bounds__(256) void permute_gather_kernel(
    const int32_t* __restrict__ perm_src, int64_t R, const uint8_t* __restrict__ xq,
    const float* __restrict__ xs, int64_t H, uint8_t* __restrict__ a_out,
    float* __restrict__ a_scale_out) {
  const int64_t vec_per_row = H / 16;
  const int64_t nkb = H / 128;
  const int64_t total = R * vec_per_row;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / vec_per_row, c = i - r * vec_per_row;
    const int64_t src = perm_src[r];
    *reinterpret_cast<uint4*>(a_out + r * H + c * 16) =
        *reinterpret_cast<const uint4*>(xq + src * H + c * 16);
    if (c < nkb) a_scale_out[r * nkb + c] = xs[src * nkb + c];
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  (void)k;
  if (T <= 0 || E <= 0) return 0;
  return (size_t)(ceil_div(T, PM_TOK) * E) * sizeof(int32_t);
}

extern "C" int moe_permute(const int32_t* topk_idx, const int32_t* expert_counts, int64_t T,
                           int32_t k, int32_t E, int32_t n_shared, int32_t* offsets,
                           int32_t* perm_src, int32_t* inv_perm, const uint8_t* xq,
                           const float* xs, int64_t H, uint8_t* a_out, float* a_scale_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0, "moe_permute: T=%lld < 0", (long long)T);
  MOE_INVALID(k >= 1 && k <= 8, "moe_permute: k=%d must be in [1, 8]", (int)k);
  MOE_INVALID(E >= 1 && E <= 4096, "moe_permute: E=%d must be in [1, 4096]", (int)E);
  MOE_INVALID(n_shared == 0 || n_shared == 1, "moe_permute: n_shared=%d must be 0 or 1",
              (int)n_shared);
  MOE_INVALID(T * (k + n_shared) < (1ll << 31), "moe_permute: T*(k+n_shared) must fit int32");
  MOE_INVALID(offsets && expert_counts, "moe_permute: null offsets or expert_counts");
  const bool gather = a_out != nullptr;
  if (gather) {
    MOE_INVALID(a_scale_out && xq && xs, "moe_permute: gathering needs xq, xs, a_scale_out");
    MOE_INVALID(H > 0 && H % 128 == 0, "moe_permute: H=%lld must be a positive multiple of 128",
                (long long)H);
    MOE_INVALID(((uintptr_t)xq & 15) == 0 && ((uintptr_t)a_out & 15) == 0,
                "moe_permute: xq and a_out must be 16-byte aligned");
  }
  hipStream_t st = as_stream(stream);
  const int64_t NB = ceil_div(T, PM_TOK);
  if (T > 0) {
    MOE_INVALID(topk_idx && perm_src && inv_perm, "moe_permute: null pointer");
    const size_t need = moe_permute_workspace_bytes(T, k, E);
    MOE_REQUIRE(workspace != nullptr && workspace_bytes >= need, MOE_ERR_WORKSPACE,
                "moe_permute: workspace needs %zu bytes, got %zu", need, workspace_bytes);
  }
  int32_t* hist = static_cast<int32_t*>(workspace);
  if (T > 0)
    permute_count_kernel<<<dim3((unsigned)NB), dim3(64), E * sizeof(int), st>>>(topk_idx, T, k, E,
                                                                                 hist);
  permute_scan_kernel<<<dim3((unsigned)E), dim3(256), 0, st>>>(expert_counts, E, T, k, n_shared,
                                                               NB, hist, offsets);
  if (T > 0) {
    int nbits = 1;
    while ((1 << nbits) <= E) ++nbits;  // ids 0..E (E = padding sentinel)
    permute_scatter_kernel<<<dim3((unsigned)NB), dim3(64), (E + 1) * sizeof(int), st>>>(
        topk_idx, T, k, E, nbits, hist, n_shared, perm_src, inv_perm);
    if (gather) {
      const int64_t R = T * k + n_shared * T;
      const int64_t total = R * (H / 16);
      const int64_t blocks = std::min<int64_t>(ceil_div(total, 256), 256 * 32);
      permute_gather_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(perm_src, R, xq, xs, H,
                                                                          a_out, a_scale_out);
    }
  }
  return check_launch("moe_permute");
}

extern "C" int moe_permute_noalloc(const int32_t* topk_idx, const int32_t* expert_counts,
                                   int64_t T, int32_t k, int32_t E, int32_t n_shared,
                                   int32_t* offsets, int32_t* perm_src, int32_t* inv_perm,
                                   const uint8_t* xq, const float* xs, int64_t H,
                                   uint8_t* a_out, float* a_scale_out, void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && E >= 1, "moe_permute_noalloc: T=%lld, E=%d", (long long)T, (int)E);
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  MOE_REQUIRE(need <= MOE_PERMUTE_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
              "moe_permute_noalloc: T=%lld, E=%d needs %zu bytes of scratch, more than the "
              "%zu of the static array (ceil(T/64) * E must be at most %zu)",
              (long long)T, (int)E, need, (size_t)MOE_PERMUTE_SCRATCH_BYTES,
              (size_t)MOE_PERMUTE_SCRATCH_BYTES / sizeof(int32_t));
  void* ws = scratch_address();
  if (ws == nullptr) return MOE_ERR_HIP;
  return moe_permute(topk_idx, expert_counts, T, k, E, n_shared, offsets, perm_src, inv_perm,
                     xq, xs, H, a_out, a_scale_out, ws, MOE_PERMUTE_SCRATCH_BYTES, stream);
}
