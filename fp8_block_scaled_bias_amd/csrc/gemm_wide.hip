// Block-scaled FP8 grouped GEMM for large groups: 256x256 output tiles,
// eight waves (two per SIMD), with the plain bf16 and the fused SwiGLU +
// 1x128 requantisation epilogues of gemm.hip.
//
// Method: news.qq.com/rain/a/20241229A05OQF00, section FP8 低精度训练 -
// 1x128 activation tiles and 128x128 weight blocks with fp32 scales
// (细粒度量化); MMA results accumulated in FP32 at a fixed K interval
// (提高累加精度).
//
// Per output element the result is  sum_kb S_kb * P_kb  with S_kb =
// sA[row, kb] * sB[nblk, kb] and P_kb the 128-term FP8 dot product of K
// block kb.  One accumulator per element carries the running sum in units of
// the current block's scale:
//     acc_0 = P_0,   acc_kb = acc_{kb-1} * (S_{kb-1} / S_kb) + P_kb,
//     result = acc_last * S_last.
// The rescale is one fp32 multiply per element per K block (the cost of a
// promotion FMA) and P_kb is added by the MFMAs themselves (C operand = the
// rescaled accumulator).  On gfx950 the MFMA adds its C operand to the
// product sum with one fp32 rounding at the magnitudes that occur here, so
// this keeps the MFMA block error of promoting a zero-started partial, with
// half the accumulator registers: a 64x128 tile per wave then fits two waves
// per SIMD.  The ratios S_{kb-1}/S_kb (correctly rounded fp32 division) are
// computed once per tile row and weight block by the whole workgroup and
// shared through LDS.  Scales are assumed to be normal fp32 numbers
// (amax/448 of finite data); scale products below ~1e-30 can overflow the
// rescaled accumulator.
//
// Pipeline: a step is 64 K (one v_mfma_f32_32x32x64_f8f6f4 per 32x32
// block); a ring of 4 LDS stages (A 256 x 64 B, B 256 x 64 B) is filled
// 3 steps ahead by global_load_lds_dwordx4 copies that each wave spreads over
// its MFMAs; K-block scales come 4 steps ahead, the gathered row-index table
// of a tile 7 steps ahead.  Each step waits (vmcnt) only for the copies of
// the step it is about to use.
//   step s: wait, barrier; per wave 8 MFMAs with the copies of step s+3
//   interleaved; after the second step of a K block, the ratios of the next
//   block; after the last step of a tile, the epilogue.
// Waves whose 64 rows lie past the group's end skip their MFMAs (a ragged
// last tile costs about half a tile when at most 128 rows remain).
#include "gemm_common.h"

#include <type_traits>

namespace moe {
namespace gemm {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int WT = 512;                  // 8 waves, 2 per SIMD
constexpr int WBM = 256;                 // tile rows
constexpr int A_BYTES = 256 * 64;        // A stage: 256 rows x 64 B (swizzled)
constexpr int B_BYTES = 256 * 64;        // B stage: 256 rows x 64 B
constexpr int STAGE = A_BYTES + B_BYTES;
constexpr int NSTAGE = 4;
constexpr int SSLOT = 320 * 4;           // sA[256], then sB[2] (64-float landing area)
constexpr int OFF_SC = NSTAGE * STAGE;               // 4 scale slots
constexpr int OFF_R = OFF_SC + 4 * SSLOT;            // float [2][2 halves][256 rows]
constexpr int OFF_PREF = OFF_R + 2 * 2 * 256 * 4;    // int [MAXG + 1]
constexpr int OFF_OFFS = OFF_PREF + (MAXG + 1) * 4;  // int [MAXG + 1]
constexpr int OFF_RIDX = OFF_OFFS + (MAXG + 1) * 4;  // int [4 tiles][256]
constexpr int OFF_AMAX = OFF_RIDX + 4 * 256 * 4;     // float [256][2]
constexpr int LDS = OFF_AMAX + 256 * 2 * 4;
static_assert(LDS <= 160 * 1024 - 256, "LDS budget");
static_assert(OFF_R % 16 == 0 && OFF_SC % 16 == 0 && SSLOT % 16 == 0, "float4 reads");

// 64 B rows: 16 B chunk c of row r sits in slot c ^ swz64(r).  For any 16
// consecutive rows read at one chunk (a 16-lane phase of ds_read_b128 on a
// 64-bank LDS) and any 8 consecutive rows (an 8-lane phase on 32 banks) the
// slots spread the rows over distinct banks.
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// 32 bytes (chunks 2q, 2q+1, q = lane/32) of row `row` of a 64 B-row stage:
// the A or B operand of one 32x32x64 MFMA for lane row `row`.
__device__ __forceinline__ v8i lds_frag64(const uint8_t* tile, int row, int q) {
  const int sw = swz64(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * 64 + (((2 * q) ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * 64 + (((2 * q + 1) ^ sw) << 4));
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// 32x32 output block over 64 K: lane l feeds row l%32 of A and of B (K bytes
// 32*(l/32)..+31); result element r of lane l is row 8*(r/4) + 4*(l/32) +
// r%4, column l%32.
__device__ __forceinline__ v16f mfma32(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Raw buffer resource over `bytes` bytes at p (gfx9 dword3: 32-bit data,
// no swizzle).  Stores at offsets past `bytes` are dropped by the hardware,
// which masks rows past a group's end without per-lane tests; the lane part
// of an address is one VGPR, the rest an SGPR offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Position of a step in this workgroup's step sequence: tile ordinal and
// step within the tile (2 per K block).
struct Cursor {
  int ord, k;
  __device__ __forceinline__ void next(int spt) {
    if (++k == spt) { k = 0; ++ord; }
  }
};

template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(WT, 1) void wide_gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  __shared__ int s_red[8];
  __shared__ int s_carry;
  int* s_pref = reinterpret_cast<int*>(smem + OFF_PREF);
  int* s_offs = reinterpret_cast<int*>(smem + OFF_OFFS);
  const int* s_ridx = reinterpret_cast<const int*>(smem + OFF_RIDX);
  float* s_r = reinterpret_cast<float*>(smem + OFF_R);
  float* s_amax = reinterpret_cast<float*>(smem + OFF_AMAX);
  const float* s_sc = reinterpret_cast<const float*>(smem + OFF_SC);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;  // wave tile: rows 64*wm.., columns 128*wn..
  const int q = lane >> 5, l32 = lane & 31;
  const int G = args.G;
  const int64_t K = args.K, N = args.N, ntiles = args.ntiles;
  const int nkb = (int)(K >> 7);  // even, >= 4 (host)
  const int spt = 2 * nkb;        // steps per tile, a multiple of 4
  const int64_t nblk = N >> 7;

  build_group_tables<WT, WBM>(args.offs, G, s_offs, s_pref, s_red, &s_carry);
  const int64_t total = (int64_t)s_pref[G] * ntiles;
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3, nper = gridDim.x >> 3;
  const int64_t chunk = (total + 7) >> 3;
  const int64_t tlo = xcd * chunk, thi = min(total, tlo + chunk);
  const int64_t L0 = tlo + jw;
  if (L0 >= thi) return;
  const int my_n = (int)((thi - L0 + nper - 1) / nper);

  // tile ordinal -> tile.  Tile ids of this workgroup increase with the
  // ordinal, so each user keeps the group of its last tile as a hint and
  // scans forward from it (empty groups are skipped).
  auto tile_at = [&](int& gh, int ord) {
    const int64_t L = L0 + (int64_t)ord * nper;
    int g = gh;
    while (g + 1 < G && (int64_t)s_pref[g + 1] * ntiles <= L) ++g;
    g = __builtin_amdgcn_readfirstlane(g);
    gh = g;
    Tile t;
    const uint32_t cnt = (uint32_t)(s_pref[g + 1] - s_pref[g]);
    const uint32_t rem = (uint32_t)(L - (int64_t)s_pref[g] * ntiles);
    const uint32_t nt = rem / cnt;
    t.g = g;
    t.nt = __builtin_amdgcn_readfirstlane((int)nt);
    t.m0 = __builtin_amdgcn_readfirstlane(s_offs[g] + (int)(rem - nt * cnt) * WBM);
    t.m1 = __builtin_amdgcn_readfirstlane(s_offs[g + 1]);
    return t;
  };
  int gh = __builtin_amdgcn_readfirstlane(decode_tile(s_pref, s_offs, G, ntiles, L0, WBM).g);
  // weight block (of 128 columns) of the tile's column half b
  auto nblk_of = [&](const Tile& t, int b) -> int64_t {
    return SWIGLU ? (b ? (args.I >> 7) + t.nt : t.nt) : 2 * t.nt + b;
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- copy sources of one tile (per lane).  Tile copy instruction p
  // (0..15) of a stage half covers rows 16p..16p+15: lane -> row 16p +
  // lane/4, LDS slot lane%4, global chunk (lane%4) ^ swz64(row); wave wv
  // issues p = 2wv, 2wv+1 for A and for B.  Scales: waves 0-3 copy sA of 64
  // rows each, wave 4 the two sB of the tile.  Gathered A rows come from
  // the tile's row-index table in LDS (buffer ord & 3).
  struct Srcs {
    const uint8_t* a0;
    const uint8_t* a1;
    const uint8_t* b0;  // B rows of p = 2wv; p = 2wv + 1 is 16 rows further
    const float* sc;
  };
  auto make_srcs = [&](const Tile& t, int ord) {
    Srcs r;
    const uint8_t* ap[2];
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
      const int row = 32 * wv + 16 * pi + (lane >> 2);
      const int gch = (lane & 3) ^ swz64(row);
      const int64_t ar = GATHER ? (int64_t)s_ridx[(ord & 3) * 256 + row] : (int64_t)min(t.m0 + row, t.m1 - 1);
      ap[pi] = args.A + ar * K + gch * 16;
    }
    r.a0 = ap[0];
    r.a1 = ap[1];
    {
      const int row = 32 * wv + (lane >> 2);
      const int gch = (lane & 3) ^ swz64(row);
      int64_t n;
      if (SWIGLU) n = (row < 128 ? 0 : args.I - 128) + 128 * t.nt + row;
      else n = 256 * t.nt + row;
      r.b0 = args.B + ((int64_t)t.g * N + n) * K + gch * 16;
    }
    if (wv < 4) {
      const int row = 64 * wv + lane;
      const int64_t ar = GATHER ? (int64_t)s_ridx[(ord & 3) * 256 + row] : (int64_t)min(t.m0 + row, t.m1 - 1);
      r.sc = args.A_scale + ar * nkb;
    } else {
      r.sc = args.B_scale + ((int64_t)t.g * nblk + nblk_of(t, lane == 1)) * nkb;
    }
    return r;
  };
  const uint32_t m0_w = lds0 + (uint32_t)(2 * wv) * 1024;  // this wave's first copy slot
  // tile copy op (0, 1: A rows p = 2wv, 2wv+1; 2, 3: B rows) of tile step kk into stage st
  auto tile_op = [&](const Srcs& r, int op, int kk, int st) {
    const uint32_t dst = m0_w + (uint32_t)st * STAGE + ((op & 2) ? A_BYTES : 0) + (op & 1) * 1024;
    const int64_t ko = (int64_t)kk * 64;
    const uint8_t* src = (op == 0) ? r.a0 : (op == 1) ? r.a1 : (op == 2) ? r.b0 : r.b0 + 16 * K;
    dma16(src + ko, dst);
  };
  auto scale_op = [&](const Srcs& r, int kb, int gslot) {
    const uint32_t ss = lds0 + OFF_SC + (uint32_t)gslot * SSLOT;
    if (wv < 4) dma4(r.sc + kb, ss + wv * 256);
    else if (wv == 4) dma4(r.sc + kb, ss + 1024);
  };
  // row-index table of a tile: waves 4-7, 64 rows each
  auto table_src = [&](const Tile& t) -> const int32_t* {
    return args.a_row_index + min(t.m0 + 64 * (wv - 4) + lane, t.m1 - 1);
  };
  auto table_op = [&](const int32_t* src, int ord) {
    dma4(src, lds0 + OFF_RIDX + (uint32_t)(((ord & 3) * 256 + 64 * (wv - 4)) * 4));
  };
  // copies per step of this wave in steady state (vmcnt bookkeeping)
  const int n_step = 4 + (wv <= 4 ? 1 : 0) + (GATHER && wv >= 4 ? 1 : 0);

  // ---- prologue: table of tile 0, then its first 3 steps and the scales
  // of its first 2 K blocks; all waited for.
  Tile tc = tile_at(gh, 0);
  const int32_t* tb_src = nullptr;
  if (GATHER) {
    if (wv >= 4) {
      tb_src = table_src(tc);
      table_op(tb_src, 0);
    }
    wait_vm_lgkm0();
    barrier();
  }
  Srcs cur = make_srcs(tc, 0);
#pragma unroll
  for (int kk = 0; kk < 3; ++kk)
#pragma unroll
    for (int op = 0; op < 4; ++op) tile_op(cur, op, kk, kk);
  scale_op(cur, 0, 0);
  scale_op(cur, 1, 1);
  scale_op(cur, 2, 2);
  wait_vm_lgkm0();
  barrier();

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS operand reads: lane-constant offsets of the two 16 B chunks of its
  // 32 B K slice (rows are multiples of 32 plus l32, so swz64 depends on l32
  // only); everything else is a compile-time offset.  Stages 2, 3 use a
  // second base so that immediate offsets stay below 64 KiB.
  const int sw = swz64(l32);
  const uint32_t o_lo = (uint32_t)(l32 * 64 + (((2 * q) ^ sw) << 4));
  const uint32_t o_hi = (uint32_t)(l32 * 64 + (((2 * q + 1) ^ sw) << 4));
  const uint8_t* pa_lo = smem + wm * 64 * 64 + o_lo;
  const uint8_t* pa_hi = smem + wm * 64 * 64 + o_hi;
  const uint8_t* pb_lo = smem + A_BYTES + (SWIGLU ? wn * 64 : wn * 128) * 64 + o_lo;
  const uint8_t* pb_hi = smem + A_BYTES + (SWIGLU ? wn * 64 : wn * 128) * 64 + o_hi;
  auto read_frag = [&](const uint8_t* lo, const uint8_t* hi, int off) -> v8i {
    const uint4 a = *reinterpret_cast<const uint4*>(lo + off);
    const uint4 b = *reinterpret_cast<const uint4*>(hi + off);
    v8i r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
  };
  // B stage row offset (from the wave's base row) of column block j
  auto b_roff = [&](int j) -> int { return SWIGLU ? (j < 2 ? 32 * j : 128 + 32 * (j - 2)) : 32 * j; };
  auto half_of = [&](int j) -> int { return SWIGLU ? (j >= 2) : wn; };

  bool drain = false;  // stores pending: the next wait is for everything
  int gh_n = gh;       // hint for decoding the next tile
  Tile tn = tc;

  for (int ord = 0; ord < my_n; ++ord) {
    const bool has_next = ord + 1 < my_n;
    const bool wvalid = tc.m0 + 64 * wm < tc.m1;
    const int gbase = ord * nkb;  // global K-block index of this tile's kb 0

    // one step k = k4 + U of this tile (stage U: tiles start at a multiple
    // of 4 steps; K block k4/2 + U/2, ratio buffer (U/2) ^ 1 after it)
    auto step = [&](auto U_, int k4) {
      constexpr int U = decltype(U_)::value;
      const int k = k4 + U;
      // copies of step k are done (those of the next two steps may still
      // fly; after stores and at the end of the work, everything); then
      // everyone is past the previous step
      if (drain || (!has_next && k + 6 >= spt)) wait_vm_lgkm0();
      else if (n_step == 4) wait_vmcnt_lgkm0<8>();
      else if (n_step == 5) wait_vmcnt_lgkm0<10>();
      else wait_vmcnt_lgkm0<12>();
      drain = false;
      barrier();

      // ---- next tile's table (8 steps ahead) and decode
      if (has_next) {
        if (GATHER && k == spt - 8) {
          tn = tile_at(gh_n, ord + 1);
          if (wv >= 4) tb_src = table_src(tn);
        }
        if (!GATHER && k == spt - 5) tn = tile_at(gh_n, ord + 1);
      }
      // ---- scales of the K block of step k+5 (re-copied: same data)
      {
        const int kb5 = (k + 5) >> 1;
        if (kb5 < nkb) scale_op(cur, kb5, (gbase + kb5) & 3);
        else if (has_next) scale_op(make_srcs(tn, ord + 1), kb5 - nkb, (gbase + kb5) & 3);
      }
      // ---- the current or next tile's row-index table (re-copied)
      if (GATHER && wv >= 4 && (has_next || k + 8 < spt))
        table_op(tb_src, (GATHER && has_next && k >= spt - 8) ? ord + 1 : ord);
      // ---- tile copies of step k+3 ride between the MFMAs below
      // (the last 3 steps copy the next tile's first steps; its sources are
      // formed for those few steps only)
      const bool t_cur = k + 3 < spt;
      const bool do_t = t_cur || has_next;
      const int kt = t_cur ? k + 3 : k + 3 - spt;
      const Srcs ts = t_cur ? cur : make_srcs(tn, ord + 1);
      constexpr int ST = U;                   // stage of step k
      constexpr int SOFF = (ST & 1) * STAGE;  // offset within the stage pair
      constexpr int TST = (U + 3) & 3;        // stage of step k+3

      const int kb = (k4 >> 1) + (U >> 1);
      if (wvalid) {
        const uint8_t* alo = pa_lo + (ST >= 2 ? 2 * STAGE : 0);
        const uint8_t* ahi = pa_hi + (ST >= 2 ? 2 * STAGE : 0);
        const uint8_t* blo = pb_lo + (ST >= 2 ? 2 * STAGE : 0);
        const uint8_t* bhi = pb_hi + (ST >= 2 ? 2 * STAGE : 0);
        v8i a[2], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = read_frag(alo, ahi, SOFF + i * 32 * 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = read_frag(blo, bhi, SOFF + b_roff(j) * 64);
        // rescale by S_kb-1 / S_kb in two halves: column blocks 2, 3 here
        // (first step of K block kb, between the MFMAs of blocks 0, 1 and
        // their own), blocks 0, 1 at the end of the previous step; each step
        // then carries half of the multiplies
        float rr[2][16];
        auto load_ratios = [&](int kbr, int hb) __attribute__((always_inline)) {
          const float* rsh = s_r + (kbr & 1) * 512 + hb * 256 + wm * 64 + 4 * q;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 v = *reinterpret_cast<const float4*>(rsh + 32 * i + 8 * g);
              rr[i][4 * g] = v.x; rr[i][4 * g + 1] = v.y;
              rr[i][4 * g + 2] = v.z; rr[i][4 * g + 3] = v.w;
            }
        };
        auto rescale_block = [&](int j) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] *= rr[i][r];
        };
        const bool resc_now = (U & 1) == 0 && kb > 0;           // blocks 2, 3, ratio of kb
        const bool resc_next = (U & 1) == 1 && kb + 1 < nkb;    // blocks 0, 1, ratio of kb+1
        if (resc_now) load_ratios(kb, SWIGLU ? 1 : wn);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (resc_now && j >= 2) rescale_block(j);
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
          if (do_t) tile_op(ts, j, kt, TST);
        }
        if (resc_next) {
          load_ratios(kb + 1, SWIGLU ? 0 : wn);
          rescale_block(0);
          rescale_block(1);
        }
      } else if (do_t) {
#pragma unroll
        for (int op = 0; op < 4; ++op) tile_op(ts, op, kt, TST);
      }

      // ---- after a K block's first step: ratios S_kb / S_kb+1 for the
      // next block of the same tile (used from the next step on)
      if ((U & 1) == 0 && kb + 1 < nkb) {
        const float* sc0 = s_sc + ((gbase + kb) & 3) * (SSLOT / 4);
        const float* sc1 = s_sc + ((gbase + kb + 1) & 3) * (SSLOT / 4);
        const int row = tid & 255, b = tid >> 8;
        const float S0 = sc0[row] * sc0[256 + b];
        const float S1 = sc1[row] * sc1[256 + b];
        s_r[((kb + 1) & 1) * 512 + b * 256 + row] = S0 / S1;
      }
    };
    for (int k4 = 0; k4 < spt; k4 += 4) {
      step(std::integral_constant<int, 0>(), k4);
      step(std::integral_constant<int, 1>(), k4);
      step(std::integral_constant<int, 2>(), k4);
      step(std::integral_constant<int, 3>(), k4);
    }

    // ---- epilogue of tile ord: result = acc * S_last ----
    const Tile t = tc;
    const float* scl = s_sc + ((gbase + nkb - 1) & 3) * (SSLOT / 4);
    // lane row of element r of row block i: 32i + 8(r/4) + 4q + r%4
    if (wvalid) {
      const float sb[2] = {scl[256], scl[257]};
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 v = *reinterpret_cast<const float4*>(scl + wm * 64 + 32 * i + 8 * g + 4 * q);
          const float sa[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[i][j][4 * g + p] *= sa[p] * sb[half_of(j)];
        }
    }
    if (!SWIGLU) {
      // bf16 (round to nearest even); lane 4k of a quad stores the 4
      // consecutive columns of lanes 4k..4k+3 as one 8-byte word
      if (wvalid) {
        const uint32_t rowb = (uint32_t)N * 2;
        const __amdgpu_buffer_rsrc_t rs =
            out_rsrc(args.C + (int64_t)t.m0 * N, (uint32_t)min(t.m1 - t.m0, WBM) * rowb);
        const int vb = (wm * 64 + 4 * q) * (int)rowb + (int)(256 * t.nt + wn * 128 + l32) * 2;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float v0 = acc[i][j][r];
              const float v1 = quad_lane1(v0), v2 = quad_lane2(v0), v3 = quad_lane3(v0);
              const int so = (32 * i + 8 * (r >> 2) + (r & 3)) * (int)rowb + 64 * j;
              if ((lane & 3) == 0) {
                typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                const v2u w = {f32x2_to_bf16x2(v0, v1), f32x2_to_bf16x2(v2, v3)};
                __builtin_amdgcn_raw_buffer_store_b64(w, rs, vb, so, 0);
              }
            }
          }
      }
    } else {
      // h = silu(g) * u: gate block j pairs with up block j + 2 in this
      // lane's registers; a row's 128 h columns are split over the two
      // column waves, whose row maxima meet in LDS.
      if (wvalid) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float g = acc[i][j][r], u = acc[i][j + 2][r];
              const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
              acc[i][j][r] = g * __builtin_amdgcn_rcpf(1.0f + e) * u;
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float m = fmaxf(fabsf(acc[i][0][r]), fabsf(acc[i][1][r]));
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
            if (l32 == 0) s_amax[(wm * 64 + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3)) * 2 + wn] = m;
          }
      }
      wait_lgkm0();
      barrier();
      if (wvalid) {
        const int I = (int)args.I, hb = I >> 7;
        const uint32_t rows = (uint32_t)min(t.m1 - t.m0, WBM);
        const __amdgpu_buffer_rsrc_t rq = out_rsrc(args.Hq + (int64_t)t.m0 * I, rows * I);
        const __amdgpu_buffer_rsrc_t rsc = out_rsrc(args.Hs + (int64_t)t.m0 * hb, rows * hb * 4);
        const int vq = (wm * 64 + 4 * q) * I + (int)(128 * t.nt) + wn * 64 + l32;
        const int vs = ((wm * 64 + 4 * q) * hb + (int)t.nt) * 4;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = 32 * i + 8 * (r >> 2) + (r & 3);  // row in the wave's 64, less 4q
            const int trow = wm * 64 + rl + 4 * q;
            const float amax = fmaxf(s_amax[trow * 2], s_amax[trow * 2 + 1]);
            const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
            const float inv = 1.0f / sc;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float v0 = acc[i][j][r] * inv;
              const float v1 = quad_lane1(v0), v2 = quad_lane2(v0), v3 = quad_lane3(v0);
              if ((lane & 3) == 0)
                __builtin_amdgcn_raw_buffer_store_b32(f32x4_to_e4m3x4(v0, v1, v2, v3), rq, vq,
                                                      rl * I + 32 * j, 0);
            }
            if (wn == 0 && l32 == 0)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsc, vs, rl * hb * 4, 0);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    drain = true;  // the stores count in vmcnt and may finish out of order
    if (has_next) {
      tc = tn;
      cur = make_srcs(tc, ord + 1);
    }
  }
}

}  // namespace

int launch_wide(const GemmArgs& a, bool swiglu, hipStream_t st) {
  const int grid = std::max(8, (num_cus() / 8) * 8);
  if (swiglu) {
    if (a.a_row_index) wide_gemm_kernel<true, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
    else wide_gemm_kernel<true, false><<<dim3(grid), dim3(WT), 0, st>>>(a);
  } else {
    if (a.a_row_index) wide_gemm_kernel<false, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
    else wide_gemm_kernel<false, false><<<dim3(grid), dim3(WT), 0, st>>>(a);
  }
  return MOE_OK;
}

}  // namespace gemm
}  // namespace moe
