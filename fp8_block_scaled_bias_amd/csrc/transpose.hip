// Transpose of FP8 weights stored in 128x128 blocks: the operand of the
// expert GEMMs' input gradient.
//
// The forward product of a group is C = A W^T with W [N, K] in 128x128
// blocks, each with one fp32 scale (news.qq.com/rain/a/20241229A05OQF00,
// section FP8 低精度训练 › 细粒度量化).  Its input gradient dA = dY W (the
// "backward for input" chunks of the same article's DualPipe overlap figure,
// section 工程 › DualPipe 流水线并行) contracts over n, so the grouped GEMM
// needs W^T [K, N] as its [N', K'] operand.  A block's codes move as they are
// and its scale moves with it: the result quantises W^T with the same blocks,
// exactly.
//
// One workgroup per block (16 KB): 16 B loads of the block's 128 rows into
// LDS (row pitch 33 dwords: at most 2-way bank conflicts), 4x4 byte
// transposes in registers (v_perm_b32), and stores of whole 128 B rows of
// the transposed block (32 lanes x 4 B).  HBM bound: 2 B per element.
#include "common.h"

namespace moe {
namespace {

constexpr int TP = 33;  // LDS row pitch in dwords

// c[i] byte j = r[j] byte i
__device__ __forceinline__ void transpose4x4(const uint32_t r[4], uint32_t c[4]) {
  // __builtin_amdgcn_perm(hi, lo, sel): result byte b = byte sel_b of hi:lo
  // (selectors 0-3 pick lo's bytes, 4-7 hi's)
  const uint32_t lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0.0 r1.0 r0.1 r1.1
  const uint32_t hi01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0.2 r1.2 r0.3 r1.3
  const uint32_t lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
  c[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);  // r0.0 r1.0 r2.0 r3.0
  c[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

__global__ __launch_bounds__(256) void transpose_128x128_kernel(
    const uint8_t* __restrict__ w, const float* __restrict__ ws, int64_t N, int64_t K,
    uint8_t* __restrict__ wt, float* __restrict__ wts) {
  __shared__ uint32_t tile[128 * TP];
  const int t = threadIdx.x;
  const int64_t kb = blockIdx.x, nb = blockIdx.y, g = blockIdx.z;
  const int64_t nkb = K >> 7, nnb = N >> 7;
  // block rows n = t/8 + 32i, 16 B chunk t%8 of each
  const uint8_t* src = w + (g * N + nb * 128) * K + kb * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = (t >> 3) + 32 * i, c = t & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)n * K + c * 16);
    uint32_t* d = tile + n * TP + c * 4;
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
  __syncthreads();
  // 4x4 byte blocks: rows n = 4a..4a+3, bytes k = 4b..4b+3 become rows
  // k = 4b..4b+3 of the output, bytes n = 4a..4a+3 (lanes a = 0..31 store
  // one whole 128 B output row)
  uint8_t* dst = wt + (g * K + kb * 128) * N + nb * 128;
  const int a = t & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = (t >> 5) + 8 * i;
    uint32_t r[4], c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = tile[(4 * a + j) * TP + b];
    transpose4x4(r, c);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint32_t*>(dst + (int64_t)(4 * b + j) * N + 4 * a) = c[j];
  }
  if (t == 0) wts[(g * nkb + kb) * nnb + nb] = ws[(g * nnb + nb) * nkb + kb];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int fp8_transpose_128x128(const uint8_t* w_e4m3, const float* w_scale, int64_t G,
                                     int64_t N, int64_t K, uint8_t* wt_e4m3, float* wt_scale,
                                     void* stream) {
  clear_error();
  MOE_INVALID(G >= 0 && G <= 65535, "fp8_transpose_128x128: G=%lld out of [0, 65535]",
              (long long)G);
  MOE_INVALID(N > 0 && N % 128 == 0 && K > 0 && K % 128 == 0,
              "fp8_transpose_128x128: N=%lld and K=%lld must be positive multiples of 128",
              (long long)N, (long long)K);
  MOE_INVALID(N / 128 <= 65535 && K / 128 <= (1ll << 31) - 1, "fp8_transpose_128x128: too large");
  if (G == 0) return MOE_OK;
  MOE_INVALID(w_e4m3 && w_scale && wt_e4m3 && wt_scale, "fp8_transpose_128x128: null pointer");
  MOE_INVALID(((uintptr_t)w_e4m3 & 15) == 0 && ((uintptr_t)wt_e4m3 & 3) == 0 &&
                  ((uintptr_t)w_scale & 3) == 0 && ((uintptr_t)wt_scale & 3) == 0,
              "fp8_transpose_128x128: w must be 16-byte, wt and the scales 4-byte aligned");
  MOE_INVALID((const void*)w_e4m3 != (const void*)wt_e4m3 && (const void*)w_scale != (const void*)wt_scale,
              "fp8_transpose_128x128: outputs must not alias the inputs");
  transpose_128x128_kernel<<<dim3((unsigned)(K / 128), (unsigned)(N / 128), (unsigned)G), dim3(256),
                             0, as_stream(stream)>>>(w_e4m3, w_scale, N, K, wt_e4m3, wt_scale);
  return check_launch("fp8_transpose_128x128");
}
