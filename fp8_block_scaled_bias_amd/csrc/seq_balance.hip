// Sequence-wise balance statistic of the router's choice.
//
// Method: news.qq.com/rain/a/20241229A05OQF00, section 无额外损耗的负载均衡
// (the sequence-level balance factor alpha = 0.0001), and the V3 summary at
// m.jxzklqfsx.com/aigc/3586.html, section （二）無輔助損失負載均衡策略革新 (a
// sequence-level term that guards against imbalance inside one sequence,
// next to the bias).  The pages print no formula; the form computed here:
// for a sequence of L consecutive tokens, with s the unbiased sigmoid scores
// of all E routed experts and S = sum_e s per token,
//   P_e = (1/L) sum_t s[t,e] / S[t],
//   f_e = E / (k L) * (number of the sequence's tokens that chose e),
//   L_bal = alpha * sum_e f_e P_e.
// The last sequence may be shorter than seq_len.
//
// Two kernels, every sum in a fixed order (results do not depend on the
// schedule):
//  1. seq_balance_partial: one workgroup per (sequence, 64-token chunk);
//     thread e adds s[t,e] / S[t] over the chunk's tokens in order, and the
//     chunk's choices are counted with LDS integer atomics;
//  2. seq_balance_final: one workgroup per sequence adds its chunks in order
//     and reduces f_e P_e over the experts (a wave butterfly, then the four
//     waves in order).
#include "common.h"

namespace moe {
namespace {

constexpr int SB_TOK = 64;

__global__ __launch_bounds__(256) void seq_balance_partial_kernel(
    const float* __restrict__ scores, const float* __restrict__ ssum,
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int64_t L, int nch,
    float* __restrict__ part_p, int32_t* __restrict__ part_c) {
  __shared__ int hist[256];
  const int e = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int c = blockIdx.y;
  const int64_t t0 = b * L + (int64_t)c * SB_TOK;
  const int64_t t1 = std::min(std::min(t0 + SB_TOK, (b + 1) * L), T);
  hist[e] = 0;
  __syncthreads();
  const int n = t1 > t0 ? (int)(t1 - t0) : 0;
  for (int i = e; i < n * k; i += 256) {
    const int v = idx[t0 * k + i];
    if ((unsigned)v < (unsigned)E) atomicAdd(&hist[v], 1);
  }
  float p = 0.f;
  if (e < E)
    for (int64_t t = t0; t < t1; ++t) p += scores[t * E + e] / ssum[t];
  __syncthreads();
  if (e < E) {
    const int64_t o = (b * nch + c) * E + e;
    part_p[o] = p;
    part_c[o] = hist[e];
  }
}

__global__ __launch_bounds__(256) void seq_balance_final_kernel(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c, int64_t T, int E, int k,
    int64_t L, int nch, float alpha, float* __restrict__ f_out, float* __restrict__ p_out,
    float* __restrict__ loss_out) {
  __shared__ float red[4];
  const int e = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t Lb = std::min(L, T - b * L);
  float term = 0.f;
  if (e < E) {
    float p = 0.f;
    int cnt = 0;
    for (int c = 0; c < nch; ++c) {
      const int64_t o = (b * nch + c) * E + e;
      p += part_p[o];
      cnt += part_c[o];
    }
    p = p / (float)Lb;
    const float f = (float)((int64_t)E * cnt) / (float)((int64_t)k * Lb);
    f_out[b * E + e] = f;
    p_out[b * E + e] = p;
    term = f * p;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) term += __shfl_xor(term, o, 64);
  if ((e & 63) == 0) red[e >> 6] = term;
  __syncthreads();
  if (e == 0) loss_out[b] = alpha * ((red[0] + red[1]) + (red[2] + red[3]));
}

size_t seq_ws_half(int64_t T, int32_t E, int64_t L) {
  const int64_t B = ceil_div(T, L);
  const int64_t nch = ceil_div(std::min(L, T), (int64_t)SB_TOK);
  return ((size_t)(B * nch * E) * 4 + 255) / 256 * 256;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_seq_balance_workspace_bytes(int64_t T, int32_t E, int64_t seq_len) {
  if (T <= 0 || E <= 0 || seq_len <= 0) return 0;
  return 2 * seq_ws_half(T, E, seq_len);
}

extern "C" int moe_seq_balance(const float* scores, const float* score_sums,
                               const int32_t* topk_idx, int64_t T, int32_t E, int32_t k,
                               int64_t seq_len, float alpha, float* f_out, float* p_out,
                               float* loss_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  clear_error();
  MOE_INVALID(T >= 0 && T < (1ll << 31), "moe_seq_balance: T=%lld out of range", (long long)T);
  MOE_INVALID(E >= 1 && E <= 256, "moe_seq_balance: E=%d must be in [1, 256]", (int)E);
  MOE_INVALID(k >= 1 && k <= E, "moe_seq_balance: k=%d must be in [1, E]", (int)k);
  MOE_INVALID(seq_len >= 1 && seq_len <= 65536,
              "moe_seq_balance: seq_len=%lld must be in [1, 65536]", (long long)seq_len);
  if (T == 0) return MOE_OK;
  MOE_INVALID(scores && score_sums && topk_idx && f_out && p_out && loss_out,
              "moe_seq_balance: null pointer");
  const size_t need = moe_seq_balance_workspace_bytes(T, E, seq_len);
  MOE_REQUIRE(workspace != nullptr && workspace_bytes >= need && ((uintptr_t)workspace & 15) == 0,
              MOE_ERR_WORKSPACE, "moe_seq_balance: workspace needs %zu bytes (16-byte aligned), got %zu",
              need, workspace_bytes);
  const int64_t B = ceil_div(T, seq_len);
  const int nch = (int)ceil_div(std::min(seq_len, T), (int64_t)SB_TOK);
  float* part_p = static_cast<float*>(workspace);
  int32_t* part_c = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                               seq_ws_half(T, E, seq_len));
  hipStream_t st = as_stream(stream);
  seq_balance_partial_kernel<<<dim3((unsigned)B, (unsigned)nch), dim3(256), 0, st>>>(
      scores, score_sums, topk_idx, T, E, k, seq_len, nch, part_p, part_c);
  seq_balance_final_kernel<<<dim3((unsigned)B), dim3(256), 0, st>>>(
      part_p, part_c, T, E, k, seq_len, nch, alpha, f_out, p_out, loss_out);
  return check_launch("moe_seq_balance");
}
