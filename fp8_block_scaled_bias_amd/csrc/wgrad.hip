// Weight gradient of the expert GEMMs in FP8: dW_g = dY_g^T A_g over each
// expert's tokens (the "backward for weights" chunks of the DualPipe overlap
// figure, news.qq.com/rain/a/20241229A05OQF00, section 工程 › DualPipe
// 流水线并行; FP8 compute with fine-grained scales and FP32 accumulation,
// section FP8 低精度训练).
//
// The contraction runs over tokens, so both operands are quantised with one
// scale per 128 tokens of one column: the 1x128 tile of the transposed
// matrix (the pages give 1x128 activation tiles without the backward
// orientation; this is the reading used).  fp8_quant_128x1_grouped writes
// them chunk-major - [chunk][column][128 tokens], every group padded to
// whole 128-token chunks, so the 128 columns of one chunk that a tile reads
// are one contiguous 16 KB block - and grouped_fp8_wgrad multiplies them
// group by group:
// each chunk is one FP8 MFMA partial in FP32, carried into the FP32 total at
// its two scales (the pages' accumulation at a fixed K interval).
#include "gemm_common.h"

namespace moe {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
using gemm::v8i;

// ---- quantiser ---------------------------------------------------------------
// One workgroup per (token chunk, 128 columns).  The chunk's rows come into
// LDS by 16 B loads (16 lanes per 256 B row piece; rows past the group's end
// read as zero; with a row index, layout row r reads input row
// row_index[r], clamped to the input); then thread t owns column t % 128 and rows 64 (t / 128) ..
// +63, read from LDS (consecutive lanes, consecutive columns), and the
// workgroup writes one contiguous 16 KB block of codes.
constexpr int QT = 256;
constexpr int QP = 136;  // LDS row pitch in bf16 (272 B: 16 B aligned rows)

__global__ __launch_bounds__(QT) void quant_128x1_grouped_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ row_index,
    int64_t in_rows, const int32_t* __restrict__ offs, int G, int64_t C, uint8_t* __restrict__ out,
    float* __restrict__ scales) {
  // the group tables take 2 (G + 1) ints of dynamic LDS (sized at launch),
  // which keeps four workgroups per CU
  extern __shared__ int s_tab[];
  int* s_offs = s_tab;
  int* s_pref = s_tab + (G + 1);
  __shared__ int s_red[QT / 64];
  __shared__ int s_carry;
  __shared__ float s_amax[128];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[128 * QP];
  gemm::build_group_tables<QT, 128>(offs, G, s_offs, s_pref, s_red, &s_carry);
  const int64_t L = blockIdx.x;  // chunk
  if (L >= s_pref[G]) return;
  const gemm::Tile t = gemm::decode_tile(s_pref, s_offs, G, 1, L, 128);
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * 128;
  {
    const int piece = tid & 15;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = (tid >> 4) + 16 * it;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t.m0 + row < t.m1) {
        const int64_t src = row_index ? (int64_t)min((uint32_t)row_index[t.m0 + row], (uint32_t)(in_rows - 1))
                                      : (int64_t)(t.m0 + row);
        v = *reinterpret_cast<const uint4*>(in + src * ld_in + c0 + piece * 8);
      }
      *reinterpret_cast<uint4*>(&s_x[row * QP + piece * 8]) = v;
    }
  }
  __syncthreads();
  const int col = tid & 127, half = tid >> 7;
  float v[64];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    v[i] = bf16_to_f32(s_x[(64 * half + i) * QP + col]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  if (half) s_amax[col] = amax;
  __syncthreads();
  if (!half) s_amax[col] = fmaxf(amax, s_amax[col]);
  __syncthreads();
  amax = s_amax[col];
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  uint8_t* dst = out + (L * C + c0 + col) * 128 + 64 * half;
  auto emit = [&](auto dv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 64; i += 16) {
      uint4 w;
      w.x = f32x4_to_e4m3x4(dv(v[i]), dv(v[i + 1]), dv(v[i + 2]), dv(v[i + 3]));
      w.y = f32x4_to_e4m3x4(dv(v[i + 4]), dv(v[i + 5]), dv(v[i + 6]), dv(v[i + 7]));
      w.z = f32x4_to_e4m3x4(dv(v[i + 8]), dv(v[i + 9]), dv(v[i + 10]), dv(v[i + 11]));
      w.w = f32x4_to_e4m3x4(dv(v[i + 12]), dv(v[i + 13]), dv(v[i + 14]), dv(v[i + 15]));
      *reinterpret_cast<uint4*>(dst + i) = w;
    }
  };
  if (recip_ok(s)) {
    const float y = 1.0f / s;
    emit([&](float x) { return div_recip(x, s, y); });
  } else {
    emit([&](float x) { return x / s; });
  }
  if (!half) scales[L * C + c0 + col] = s;
}

// Without a row index (rows in layout order) the LDS staging is skipped:
// wave w takes rows 32w..32w+31 of the chunk and lane l columns 2l, 2l+1,
// one 4-byte load per row (a wave reads a whole 256 B row piece per load);
// the four waves' column maxima meet in 2 KB of LDS.  Five workgroups per CU
// instead of four, 25 % faster on such operands; gathered rows keep the
// staged kernel above (scattered 256 B rows: whole-row loads there were
// 25 % slower).
__global__ __launch_bounds__(QT) void quant_128x1_direct_kernel(
    const uint16_t* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ row_index,
    int64_t in_rows, const int32_t* __restrict__ offs, int G, int64_t C, uint8_t* __restrict__ out,
    float* __restrict__ scales) {
  // the group tables take 2 (G + 1) ints of dynamic LDS (sized at launch),
  // which keeps four workgroups per CU
  extern __shared__ int s_tab[];
  int* s_offs = s_tab;
  int* s_pref = s_tab + (G + 1);
  __shared__ int s_red[QT / 64];
  __shared__ int s_carry;
  __shared__ float s_am[4][128];
  gemm::build_group_tables<QT, 128>(offs, G, s_offs, s_pref, s_red, &s_carry);
  const int64_t L = blockIdx.x;  // chunk
  if (L >= s_pref[G]) return;
  const gemm::Tile t = gemm::decode_tile(s_pref, s_offs, G, 1, L, 128);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.y * 128;
  // wave w: rows 32w..32w+31 of the chunk; lane l: columns 2l and 2l+1, one
  // 4-byte load per row (a wave reads a whole 256 B row piece per load)
  float v0[32], v1[32];
  float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * w + i;
    uint32_t pr = 0u;
    if (t.m0 + row < t.m1) {
      const int64_t src = row_index ? (int64_t)min((uint32_t)row_index[t.m0 + row], (uint32_t)(in_rows - 1))
                                    : (int64_t)(t.m0 + row);
      pr = *reinterpret_cast<const uint32_t*>(in + src * ld_in + c0 + 2 * lane);
    }
    v0[i] = bf16_to_f32(pr & 0xFFFFu);
    v1[i] = bf16_to_f32(pr >> 16);
    m0 = fmaxf(m0, fabsf(v0[i]));
    m1 = fmaxf(m1, fabsf(v1[i]));
  }
  s_am[w][2 * lane] = m0;
  s_am[w][2 * lane + 1] = m1;
  __syncthreads();
  const float a0 = fmaxf(fmaxf(s_am[0][2 * lane], s_am[1][2 * lane]), fmaxf(s_am[2][2 * lane], s_am[3][2 * lane]));
  const float a1 = fmaxf(fmaxf(s_am[0][2 * lane + 1], s_am[1][2 * lane + 1]),
                         fmaxf(s_am[2][2 * lane + 1], s_am[3][2 * lane + 1]));
  const float s0 = a0 > 0.0f ? a0 / 448.0f : 1.0f;
  const float s1 = a1 > 0.0f ? a1 / 448.0f : 1.0f;
  uint8_t* dst0 = out + (L * C + c0 + 2 * lane) * 128 + 32 * w;
  uint8_t* dst1 = dst0 + 128;
  auto emit = [&](auto d0, auto d1) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 32; i += 16) {
      uint4 q0, q1;
      q0.x = f32x4_to_e4m3x4(d0(v0[i]), d0(v0[i + 1]), d0(v0[i + 2]), d0(v0[i + 3]));
      q0.y = f32x4_to_e4m3x4(d0(v0[i + 4]), d0(v0[i + 5]), d0(v0[i + 6]), d0(v0[i + 7]));
      q0.z = f32x4_to_e4m3x4(d0(v0[i + 8]), d0(v0[i + 9]), d0(v0[i + 10]), d0(v0[i + 11]));
      q0.w = f32x4_to_e4m3x4(d0(v0[i + 12]), d0(v0[i + 13]), d0(v0[i + 14]), d0(v0[i + 15]));
      q1.x = f32x4_to_e4m3x4(d1(v1[i]), d1(v1[i + 1]), d1(v1[i + 2]), d1(v1[i + 3]));
      q1.y = f32x4_to_e4m3x4(d1(v1[i + 4]), d1(v1[i + 5]), d1(v1[i + 6]), d1(v1[i + 7]));
      q1.z = f32x4_to_e4m3x4(d1(v1[i + 8]), d1(v1[i + 9]), d1(v1[i + 10]), d1(v1[i + 11]));
      q1.w = f32x4_to_e4m3x4(d1(v1[i + 12]), d1(v1[i + 13]), d1(v1[i + 14]), d1(v1[i + 15]));
      *reinterpret_cast<uint4*>(dst0 + i) = q0;
      *reinterpret_cast<uint4*>(dst1 + i) = q1;
    }
  };
  if (recip_ok(s0) && recip_ok(s1)) {
    const float y0 = 1.0f / s0, y1 = 1.0f / s1;
    emit([&](float x) { return div_recip(x, s0, y0); }, [&](float x) { return div_recip(x, s1, y1); });
  } else {
    emit([&](float x) { return x / s0; }, [&](float x) { return x / s1; });
  }
  if (w == 0) {
    scales[L * C + c0 + 2 * lane] = s0;
    scales[L * C + c0 + 2 * lane + 1] = s1;
  }
}

// ---- SwiGLU backward in the chunk layout -----------------------------------
// The SwiGLU backward (swiglu_bwd_elem, the arithmetic of swiglu_backward)
// over each group's 128-token chunks, writing besides dGU = [dg | du] and h
// as bf16 the codes the next steps read: dGU's 1x128 codes (the input-
// gradient GEMM's operand) and the 128x1 chunk-major codes of dGU and h (the
// two weight gradients' operands, the layout of fp8_quant_128x1_grouped), all
// from the stored bf16 values, so neither is read back.  One workgroup per
// (chunk, 128 columns of I).  Lane l of wave w owns columns 8 (l % 16) .. +7
// of rows 32w + 8 (l / 16) .. +7: a row's 1x128 tile is 16 lanes (xor 1..8),
// a column's 32 rows in a wave are 4 lanes (xor 16, 32) whose 8 codes each
// are contiguous in the chunk layout, and the four waves meet in LDS.
__global__ __launch_bounds__(QT) void swiglu_backward_grouped_kernel(
    const uint16_t* __restrict__ gu, const uint16_t* __restrict__ dh,
    const int32_t* __restrict__ offs, int G, int64_t I, uint16_t* __restrict__ dgu,
    uint16_t* __restrict__ h, uint8_t* __restrict__ dgu_q, float* __restrict__ dgu_qs,
    uint8_t* __restrict__ dgu_c, float* __restrict__ dgu_cs, uint8_t* __restrict__ h_c,
    float* __restrict__ h_cs) {
  extern __shared__ int s_tab[];
  int* s_offs = s_tab;
  int* s_pref = s_tab + (G + 1);
  __shared__ int s_red[QT / 64];
  __shared__ int s_carry;
  __shared__ float s_am[4][128];
  gemm::build_group_tables<QT, 128>(offs, G, s_offs, s_pref, s_red, &s_carry);
  const int64_t L = blockIdx.x;  // chunk
  if (L >= s_pref[G]) return;
  const gemm::Tile t = gemm::decode_tile(s_pref, s_offs, G, 1, L, 128);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = lane & 15, rs = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.y * 128, I2 = 2 * I;
  const int64_t col = c0 + 8 * cg;          // this lane's first column of I
  const int row0 = 32 * w + 8 * rs;         // its first row of the chunk
  // bf16 values of dg, du, h: [row i][4 words of 2 columns]
  uint4 pg[8], pu[8], ph[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = t.m0 + row0 + i;
    const bool ok = r < t.m1;
    const int64_t rr = ok ? r : t.m0;       // a valid row; values zeroed below
    const uint4 gv = *reinterpret_cast<const uint4*>(gu + rr * I2 + col);
    const uint4 uv = *reinterpret_cast<const uint4*>(gu + rr * I2 + I + col);
    const uint4 dv = *reinterpret_cast<const uint4*>(dh + rr * I + col);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w},
                   dw_[4] = {dv.x, dv.y, dv.z, dv.w};
    uint32_t og[4], ou[4], oh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float dg0, du0, h0, dg1, du1, h1;
      swiglu_bwd_elem(bf16_to_f32(gw[q] & 0xFFFFu), bf16_to_f32(uw[q] & 0xFFFFu),
                      bf16_to_f32(dw_[q] & 0xFFFFu), &dg0, &du0, &h0);
      swiglu_bwd_elem(bf16_to_f32(gw[q] >> 16), bf16_to_f32(uw[q] >> 16), bf16_to_f32(dw_[q] >> 16),
                      &dg1, &du1, &h1);
      og[q] = ok ? f32x2_to_bf16x2(dg0, dg1) : 0u;
      ou[q] = ok ? f32x2_to_bf16x2(du0, du1) : 0u;
      oh[q] = ok ? f32x2_to_bf16x2(h0, h1) : 0u;
    }
    pg[i] = make_uint4(og[0], og[1], og[2], og[3]);
    pu[i] = make_uint4(ou[0], ou[1], ou[2], ou[3]);
    ph[i] = make_uint4(oh[0], oh[1], oh[2], oh[3]);
    if (ok && dgu) {  // the bf16 values are optional (only their codes feed the GEMMs)
      *reinterpret_cast<uint4*>(dgu + r * I2 + col) = pg[i];
      *reinterpret_cast<uint4*>(dgu + r * I2 + I + col) = pu[i];
      *reinterpret_cast<uint4*>(h + r * I + col) = ph[i];
    }
  }
  auto unpack = [](const uint4& p, float* v) {
    const uint32_t x[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32(x[q] & 0xFFFFu);
      v[2 * q + 1] = bf16_to_f32(x[q] >> 16);
    }
  };
  // dGU's 1x128 codes: a row's tile is the 16 lanes of one rs (all valid or
  // all past the group's end together)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = t.m0 + row0 + i;
    float v[8], s;
    unpack(pg[i], v);
    const uint2 qg = quant_tile_1x128(v, &s);
    if (r < t.m1) {
      *reinterpret_cast<uint2*>(dgu_q + r * I2 + col) = qg;
      if (cg == 0) dgu_qs[r * (I2 >> 7) + (c0 >> 7)] = s;
    }
    unpack(pu[i], v);
    const uint2 qu = quant_tile_1x128(v, &s);
    if (r < t.m1) {
      *reinterpret_cast<uint2*>(dgu_q + r * I2 + I + col) = qu;
      if (cg == 0) dgu_qs[r * (I2 >> 7) + ((I + c0) >> 7)] = s;
    }
  }
  // 128x1 codes of one output: a column's maximum over the lane's 8 rows,
  // the wave's 4 row groups (xor 16, 32) and the four waves (LDS); rows past
  // the group's end are the chunk's zero padding
  auto col_codes = [&](const uint4* p, uint8_t* out, float* scl, int64_t C, int64_t cbase) {
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v[8];
      unpack(p[i], v);
#pragma unroll
      for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(v[j]));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      m[j] = fmaxf(m[j], __shfl_xor(m[j], 16, 64));
      m[j] = fmaxf(m[j], __shfl_xor(m[j], 32, 64));
    }
    if (rs == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) s_am[w][8 * cg + j] = m[j];
    }
    __syncthreads();
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int cc = 8 * cg + j;
      const float a = fmaxf(fmaxf(s_am[0][cc], s_am[1][cc]), fmaxf(s_am[2][cc], s_am[3][cc]));
      sc[j] = a > 0.0f ? a / 448.0f : 1.0f;
    }
    __syncthreads();  // s_am is reused by the next output
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[8];  // column j of this lane's 8 rows
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t x[4] = {p[i].x, p[i].y, p[i].z, p[i].w};
        const uint32_t b = (j & 1) ? (x[j >> 1] >> 16) : (x[j >> 1] & 0xFFFFu);
        v[i] = bf16_to_f32(b);
      }
      uint2 qc;
      if (recip_ok(sc[j])) {
        const float y = 1.0f / sc[j];
        qc = make_uint2(f32x4_to_e4m3x4(div_recip(v[0], sc[j], y), div_recip(v[1], sc[j], y),
                                        div_recip(v[2], sc[j], y), div_recip(v[3], sc[j], y)),
                        f32x4_to_e4m3x4(div_recip(v[4], sc[j], y), div_recip(v[5], sc[j], y),
                                        div_recip(v[6], sc[j], y), div_recip(v[7], sc[j], y)));
      } else {
        qc = make_uint2(f32x4_to_e4m3x4(v[0] / sc[j], v[1] / sc[j], v[2] / sc[j], v[3] / sc[j]),
                        f32x4_to_e4m3x4(v[4] / sc[j], v[5] / sc[j], v[6] / sc[j], v[7] / sc[j]));
      }
      *reinterpret_cast<uint2*>(out + (L * C + cbase + 8 * cg + j) * 128 + row0) = qc;
      if (w == 0 && rs == 0) scl[L * C + cbase + 8 * cg + j] = sc[j];
    }
  };
  col_codes(pg, dgu_c, dgu_cs, I2, c0);
  col_codes(pu, dgu_c, dgu_cs, I2, I + c0);
  col_codes(ph, h_c, h_cs, I, c0);
}

// ---- weight-gradient GEMM ----------------------------------------------------
// One workgroup (4 waves) per 128 (n) x 128 (k) tile of one group's dW; wave
// (wm, wn) owns rows 64wm.. and columns 64wn.. as 2 x 2 blocks of
// v_mfma_f32_32x32x64_f8f6f4.  The group's 128-token chunks pass through one
// LDS stage (rows 128 B, 16 B pieces XOR-swizzled by row so the fragment
// reads are conflict-free); chunk c+1 is loaded into registers while chunk c
// is multiplied.  One FP32 accumulator per element carries the sum in units
// of the current chunk's scale product S_c = sY[n, c] sA[k, c]:
//     acc = P_c0,   acc = acc * (S_{c-1} / S_c) + P_c,   dW = acc * S_last,
// P_c the chunk's two 64-token MFMA steps (added by the MFMAs themselves).
// The ratio is taken per operand, (sY_{c-1} / sY_c) (sA_{c-1} / sA_c), one
// quotient per thread and chunk, shared through LDS.  Against a zero-started
// partial per chunk promoted by FMA this halves the accumulator registers
// (about 165 VGPRs: three waves per SIMD instead of two) and the single stage
// halves the LDS (three workgroups per CU).  Scales are normal fp32 numbers
// (amax/448 of finite data, 1 for an all-zero column); ratios beyond ~1e30
// between consecutive chunks can overflow the rescaled accumulator.
constexpr int WGT = 256;
constexpr int TILE_B = 128 * 128;

__device__ __forceinline__ v16f mfma32(const v8i& x, const v8i& y, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
}

__global__ __launch_bounds__(WGT) void wgrad_kernel(
    const uint8_t* __restrict__ yt, const float* __restrict__ ys, const uint8_t* __restrict__ at,
    const float* __restrict__ as, const int32_t* __restrict__ offs, int64_t N, int64_t K,
    float* __restrict__ dw) {
  __shared__ __attribute__((aligned(16))) uint8_t s_y[TILE_B];
  __shared__ __attribute__((aligned(16))) uint8_t s_a[TILE_B];
  __shared__ __attribute__((aligned(16))) float s_r[2][256];   // ratios: [0..127] y, [128..255] a
  __shared__ __attribute__((aligned(16))) float s_s[256];      // the current chunk's scales
  __shared__ int s_red[WGT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1, q = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.y;
  const int64_t ktiles = K >> 7;
  const int64_t n0 = (int64_t)(blockIdx.x / ktiles) * 128, k0 = (int64_t)(blockIdx.x % ktiles) * 128;
  int part = 0;
  for (int i = tid; i < g; i += WGT) part += (offs[i + 1] - offs[i] + 127) >> 7;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (lane == 0) s_red[wv] = part;
  __syncthreads();
  const int c0 = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  const int c1 = c0 + ((offs[g + 1] - offs[g] + 127) >> 7);
  const int lrow = tid >> 3, lpc = tid & 7;
  const int soff = lrow * 128 + ((lpc ^ (lrow & 7)) << 4);
  uint4 y0, y1, y2, y3, a0, a1, a2, a3;
  float rsc = 0.0f, rprev = 1.0f;
  auto ld16 = [](const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); };
  auto load = [&](int c) {
    const uint8_t* py = yt + ((int64_t)c * N + n0 + lrow) * 128 + lpc * 16;
    const uint8_t* pa = at + ((int64_t)c * K + k0 + lrow) * 128 + lpc * 16;
    y0 = ld16(py); y1 = ld16(py + 32 * 128); y2 = ld16(py + 64 * 128); y3 = ld16(py + 96 * 128);
    a0 = ld16(pa); a1 = ld16(pa + 32 * 128); a2 = ld16(pa + 64 * 128); a3 = ld16(pa + 96 * 128);
    rsc = tid < 128 ? ys[(int64_t)c * N + n0 + tid] : as[(int64_t)c * K + k0 + tid - 128];
  };
  // chunk into LDS; thread tid's scale and its ratio to the previous chunk's
  auto store = [&](int slot) {
    *reinterpret_cast<uint4*>(s_y + soff) = y0;
    *reinterpret_cast<uint4*>(s_y + soff + 32 * 128) = y1;
    *reinterpret_cast<uint4*>(s_y + soff + 64 * 128) = y2;
    *reinterpret_cast<uint4*>(s_y + soff + 96 * 128) = y3;
    *reinterpret_cast<uint4*>(s_a + soff) = a0;
    *reinterpret_cast<uint4*>(s_a + soff + 32 * 128) = a1;
    *reinterpret_cast<uint4*>(s_a + soff + 64 * 128) = a2;
    *reinterpret_cast<uint4*>(s_a + soff + 96 * 128) = a3;
    s_s[tid] = rsc;
    s_r[slot][tid] = rprev / rsc;
    rprev = rsc;
  };
  auto frag = [&](const uint8_t* base, int row, int h) -> v8i {
    const int sw = row & 7;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * 128 + (((4 * h + 2 * q) ^ sw) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * 128 + (((4 * h + 2 * q + 1) ^ sw) << 4));
    v8i r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
  };
  v16f tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.0f;
  if (c0 < c1) {
    load(c0);
    store(0);
  }
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const bool more = c + 1 < c1;
    if (more) load(c + 1);
    if (c > c0) {  // into the units of this chunk's scales: tot *= (S_prev / S_c)
      const int sl = (c - c0) & 1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float ry = s_r[sl][64 * wm + 32 * j + l32];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float4 ra = *reinterpret_cast<const float4*>(&s_r[sl][128 + 64 * wn + 32 * i + 8 * e + 4 * q]);
            tot[i][j][4 * e + 0] *= ry * ra.x;
            tot[i][j][4 * e + 1] *= ry * ra.y;
            tot[i][j][4 * e + 2] *= ry * ra.z;
            tot[i][j][4 * e + 3] *= ry * ra.w;
          }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i xa[2], yb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) xa[i] = frag(s_a, 64 * wn + 32 * i + l32, h);
#pragma unroll
      for (int j = 0; j < 2; ++j) yb[j] = frag(s_y, 64 * wm + 32 * j + l32, h);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) tot[i][j] = mfma32(xa[i], yb[j], tot[i][j]);
    }
    if (!more) break;
    __syncthreads();
    store((c + 1 - c0) & 1);
    __syncthreads();
  }
  // result = tot * S_last, stored in whole 128 B lines: per column half i,
  // each wave's 64 rows x 32 columns (8 KB) go through LDS (the operand
  // stages, free once every wave is past the last chunk; 16 B chunk c of row
  // r in slot c ^ (r & 7)) and come back 8 rows x 128 B per store
  // instruction.  dW is written once and not read here: non-temporal stores.
  float* out = dw + ((int64_t)g * N + n0) * K + k0;
  typedef float f4v __attribute__((ext_vector_type(4)));
  __syncthreads();
  uint8_t* stg = (wv < 2 ? s_y + wv * 8192 : s_a + (wv - 2) * 8192);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 32 * j + l32;
      const float sy = c0 < c1 ? s_s[64 * wm + r] : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = 64 * wn + 32 * i + 8 * e + 4 * q;
        float4 sa = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c0 < c1) sa = *reinterpret_cast<const float4*>(&s_s[128 + k]);
        *reinterpret_cast<float4*>(stg + r * 128 + (((2 * e + q) ^ (r & 7)) << 4)) =
            make_float4(tot[i][j][4 * e] * (sy * sa.x), tot[i][j][4 * e + 1] * (sy * sa.y),
                        tot[i][j][4 * e + 2] * (sy * sa.z), tot[i][j][4 * e + 3] * (sy * sa.w));
      }
    }
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int r = 8 * r8 + (lane >> 3), ch = lane & 7;
      const float4 v = *reinterpret_cast<const float4*>(stg + r * 128 + ((ch ^ (r & 7)) << 4));
      const f4v w = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(
          w, reinterpret_cast<f4v*>(out + (int64_t)(64 * wm + r) * K + 64 * wn + 32 * i + 4 * ch));
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

static int64_t chunks_needed(int64_t M_total, int32_t G) { return ceil_div(M_total, 128) + G; }

extern "C" int fp8_quant_128x1_grouped(const void* in_bf16, int64_t ld_in,
                                       const int32_t* row_index, int64_t in_rows,
                                       const int32_t* group_offsets, int32_t G, int64_t M_total,
                                       int64_t C, uint8_t* out_c, float* scales_c,
                                       int64_t chunks_cap, void* stream) {
  clear_error();
  MOE_INVALID(G >= 1, "fp8_quant_128x1_grouped: G=%d < 1", (int)G);
  MOE_UNSUPPORTED(G <= gemm::MAXG, "fp8_quant_128x1_grouped: G=%d > %d", (int)G, gemm::MAXG);
  MOE_INVALID(M_total >= 0 && M_total < (1ll << 31), "fp8_quant_128x1_grouped: M_total=%lld out of range",
              (long long)M_total);
  MOE_INVALID(C > 0 && C % 128 == 0 && C / 128 <= 65535,
              "fp8_quant_128x1_grouped: C=%lld must be a positive multiple of 128 (at most 65535*128)",
              (long long)C);
  MOE_INVALID(ld_in >= C, "fp8_quant_128x1_grouped: ld_in=%lld < C", (long long)ld_in);
  if (M_total == 0) return MOE_OK;  // every group is empty: no chunk to write
  MOE_INVALID(row_index ? (in_rows >= 1 && in_rows < (1ll << 31)) : in_rows >= M_total,
              "fp8_quant_128x1_grouped: in_rows=%lld must be >= %s and < 2^31", (long long)in_rows,
              row_index ? "1" : "M_total");
  MOE_INVALID(chunks_cap >= chunks_needed(M_total, G),
              "fp8_quant_128x1_grouped: chunks_cap=%lld < ceil(M_total/128) + G = %lld",
              (long long)chunks_cap, (long long)chunks_needed(M_total, G));
  MOE_INVALID(in_bf16 && group_offsets && out_c && scales_c, "fp8_quant_128x1_grouped: null pointer");
  MOE_INVALID(((uintptr_t)in_bf16 & 15) == 0 && ld_in % 8 == 0 && ((uintptr_t)out_c & 15) == 0 &&
                  ((uintptr_t)scales_c & 3) == 0,
              "fp8_quant_128x1_grouped: in must be 16-byte aligned with ld_in %% 8 == 0, out 16-byte, "
              "scales 4-byte aligned");
  const int64_t chunks = chunks_needed(M_total, G);
  auto kernel = row_index ? quant_128x1_grouped_kernel : quant_128x1_direct_kernel;
  kernel<<<dim3((unsigned)chunks, (unsigned)(C / 128)), dim3(QT), 2 * (G + 1) * sizeof(int),
           as_stream(stream)>>>(
      static_cast<const uint16_t*>(in_bf16), ld_in, row_index, in_rows, group_offsets, G, C, out_c,
      scales_c);
  return check_launch("fp8_quant_128x1_grouped");
}

extern "C" int swiglu_backward_grouped(const void* gu_bf16, const void* dh_bf16,
                                       const int32_t* group_offsets, int32_t G, int64_t M_total,
                                       int64_t I, void* dgu_bf16, void* h_bf16, uint8_t* dgu_e4m3,
                                       float* dgu_scale, int64_t chunks_cap, uint8_t* dgu_c,
                                       float* dgu_scale_c, uint8_t* h_c, float* h_scale_c,
                                       void* stream) {
  clear_error();
  MOE_INVALID(G >= 1, "swiglu_backward_grouped: G=%d < 1", (int)G);
  MOE_UNSUPPORTED(G <= gemm::MAXG, "swiglu_backward_grouped: G=%d > %d", (int)G, gemm::MAXG);
  MOE_INVALID(M_total >= 0 && M_total < (1ll << 31),
              "swiglu_backward_grouped: M_total=%lld out of range", (long long)M_total);
  MOE_INVALID(I > 0 && I % 128 == 0 && I / 128 <= 65535,
              "swiglu_backward_grouped: I=%lld must be a positive multiple of 128", (long long)I);
  if (M_total == 0) return MOE_OK;
  MOE_INVALID(chunks_cap >= chunks_needed(M_total, G),
              "swiglu_backward_grouped: chunks_cap=%lld < ceil(M_total/128) + G = %lld",
              (long long)chunks_cap, (long long)chunks_needed(M_total, G));
  MOE_INVALID(gu_bf16 && dh_bf16 && group_offsets && dgu_e4m3 && dgu_scale && dgu_c &&
                  dgu_scale_c && h_c && h_scale_c,
              "swiglu_backward_grouped: null pointer");
  MOE_INVALID((dgu_bf16 == nullptr) == (h_bf16 == nullptr),
              "swiglu_backward_grouped: dgu_bf16 and h_bf16 are given together or not at all");
  MOE_INVALID(((uintptr_t)gu_bf16 & 15) == 0 && ((uintptr_t)dh_bf16 & 15) == 0 &&
                  ((uintptr_t)dgu_bf16 & 15) == 0 && ((uintptr_t)h_bf16 & 15) == 0 &&
                  ((uintptr_t)dgu_e4m3 & 15) == 0 && ((uintptr_t)dgu_c & 15) == 0 &&
                  ((uintptr_t)h_c & 15) == 0 && ((uintptr_t)dgu_scale & 3) == 0 &&
                  ((uintptr_t)dgu_scale_c & 3) == 0 && ((uintptr_t)h_scale_c & 3) == 0,
              "swiglu_backward_grouped: tensors and codes must be 16-byte, scales 4-byte aligned");
  swiglu_backward_grouped_kernel<<<dim3((unsigned)chunks_needed(M_total, G), (unsigned)(I / 128)),
                                   dim3(QT), 2 * (G + 1) * sizeof(int), as_stream(stream)>>>(
      static_cast<const uint16_t*>(gu_bf16), static_cast<const uint16_t*>(dh_bf16), group_offsets,
      G, I, static_cast<uint16_t*>(dgu_bf16), static_cast<uint16_t*>(h_bf16), dgu_e4m3, dgu_scale,
      dgu_c, dgu_scale_c, h_c, h_scale_c);
  return check_launch("swiglu_backward_grouped");
}

extern "C" int grouped_fp8_wgrad(const uint8_t* dy_c, const float* dy_scale_c, const uint8_t* a_c,
                                 const float* a_scale_c, int64_t chunks_cap,
                                 const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t N,
                                 int64_t K, float* dW, void* stream) {
  clear_error();
  MOE_INVALID(G >= 1 && G <= 65535, "grouped_fp8_wgrad: G=%d out of [1, 65535]", (int)G);
  MOE_INVALID(M_total >= 0 && M_total < (1ll << 31), "grouped_fp8_wgrad: M_total=%lld out of range",
              (long long)M_total);
  MOE_INVALID(N > 0 && N % 128 == 0 && K > 0 && K % 128 == 0,
              "grouped_fp8_wgrad: N=%lld and K=%lld must be positive multiples of 128", (long long)N,
              (long long)K);
  MOE_INVALID((N / 128) * (K / 128) <= (1ll << 31) - 1, "grouped_fp8_wgrad: too many tiles");
  MOE_INVALID(chunks_cap >= chunks_needed(M_total, G),
              "grouped_fp8_wgrad: chunks_cap=%lld < ceil(M_total/128) + G = %lld", (long long)chunks_cap,
              (long long)chunks_needed(M_total, G));
  MOE_INVALID(dy_c && dy_scale_c && a_c && a_scale_c && group_offsets && dW,
              "grouped_fp8_wgrad: null pointer");
  MOE_INVALID(((uintptr_t)dy_c & 15) == 0 && ((uintptr_t)a_c & 15) == 0 && ((uintptr_t)dW & 15) == 0 &&
                  ((uintptr_t)dy_scale_c & 3) == 0 && ((uintptr_t)a_scale_c & 3) == 0,
              "grouped_fp8_wgrad: operands and dW must be 16-byte, scales 4-byte aligned");
  wgrad_kernel<<<dim3((unsigned)((N / 128) * (K / 128)), (unsigned)G), dim3(WGT), 0, as_stream(stream)>>>(
      dy_c, dy_scale_c, a_c, a_scale_c, group_offsets, N, K, dW);
  return check_launch("grouped_fp8_wgrad");
}
