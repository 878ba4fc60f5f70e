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
// block), two steps a K block.  LDS holds two K-block stages (A 256 x 128 B,
// B 256 x 128 B): while block kb is used, block kb+1 is copied into the
// other stage by buffer_load ... lds copies that each wave spreads over the
// MFMAs of kb's first step.  A copy moves 8 rows x 128 B, so every row is
// one whole cache line (half the memory requests of 64 B row pieces).
// K-block scales come 4 steps ahead, the gathered row-index table of a tile 7
// steps ahead.  Copies address memory as a per-tile buffer resource (SGPRs)
// + a per-tile lane offset (VGPR) + the K position as the SGPR soffset,
// which moves only the global address, never the LDS one; so a step spends
// no vector instructions on addressing.  Every wave issues the same copies,
// and each step waits (vmcnt) only for what it is about to use.
//   step s: wait, barrier; per wave 8 MFMAs (the first step of a K block
//   with the next block's copies interleaved); after the first step of a K
//   block, the ratios of the next block; after the last step of a tile, the
//   epilogue.
// The steps away from a tile's first 4 and last 8 carry no run-time tests.
// Waves whose 64 rows lie past the group's end skip their MFMAs (a ragged
// last tile costs about half a tile when at most 128 rows remain).
#include "gemm_common.h"

#include <type_traits>

namespace moe {
namespace gemm {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int WT = 512;                  // 8 waves, 2 per SIMD
constexpr int WBM = 256;                 // tile rows
constexpr int ST_BYTES = 256 * 128;      // one operand's K-block stage: 256 rows x 128 B
constexpr int OFF_B = 2 * ST_BYTES;      // A stages 0, 1, then B stages 0, 1
constexpr int SSLOT = 320 * 4;           // sA[256], then sB[2] (64-float landing area)
constexpr int OFF_SC = 4 * ST_BYTES;                 // 4 scale slots
constexpr int OFF_R = OFF_SC + 4 * SSLOT;            // float [2][2 halves][256 rows]
constexpr int OFF_PREF = OFF_R + 2 * 2 * 256 * 4;    // int [MAXG + 1]
constexpr int OFF_OFFS = OFF_PREF + (MAXG + 1) * 4;  // int [MAXG + 1]
constexpr int OFF_RIDX = OFF_OFFS + (MAXG + 1) * 4;  // int [4 tiles][256]
constexpr int OFF_AMAX = OFF_RIDX + 4 * 256 * 4;     // float [256][2]
constexpr int LDS = OFF_AMAX + 256 * 2 * 4;
static_assert(LDS <= 160 * 1024 - 256, "LDS budget");
static_assert(OFF_R % 16 == 0 && OFF_SC % 16 == 0 && SSLOT % 16 == 0, "float4 reads");

// 32x32 block over 64 K: lane l feeds row l%32 of x and of y (K bytes
// 32*(l/32)..+31); result element r of lane l is x row 8*(r/4) + 4*(l/32) +
// r%4 against y row l%32.  The kernel passes weights as x and tokens as y,
// so a lane holds one token row and 16 output columns: 4 runs of 4
// consecutive columns (r = 4g..4g+3 at column 8g + 4*(l/32)).
__device__ __forceinline__ v16f mfma32(const v8i& x, const v8i& y, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
}

// Raw buffer resource over `bytes` bytes at p (gfx9 dword3: 32-bit data,
// no swizzle).  Stores at offsets past `bytes` are dropped by the hardware,
// which masks rows past a group's end without per-lane tests; the lane part
// of an address is one VGPR, the rest an SGPR offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// The same descriptor as four SGPRs, for the copies below (stride 0: the
// range check is offset < bytes; loads past it return zeros).
__device__ __forceinline__ v4i load_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Asynchronous copies into LDS.  Lane i's 16 (4) bytes come from buffer
// offset voff + soff and land at m0 + i*16 (i*4); soff moves the global
// address only.  m0 and soff must be wave-uniform (SGPRs).
template <int IMM>
__device__ __forceinline__ void copy16(const v4i& r, uint32_t voff, uint32_t soff, uint32_t m0b) {
  asm volatile("s_add_u32 m0, %3, %4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(r), "s"(soff), "s"(m0b), "n"(IMM)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ void copy4(const v4i& r, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               ::"v"(voff), "s"(r), "s"(soff), "s"(m0)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

template <int V>
using ic = std::integral_constant<int, V>;

// Estimated cost of a tile in 1/20 of a full one (timed per tile): a group's
// last tile copies all of B but only its own A rows, and the waves past its
// rows skip their MFMAs.
constexpr int COST_FULL = 20;
__device__ __forceinline__ int last_tile_cost(int rem) {
  return rem == 0 ? 0 : rem <= 64 ? 14 : rem <= 128 ? 15 : rem <= 192 ? 19 : COST_FULL;
}

// s_cpref[0..G] = exclusive prefix over groups of the cost of one N-tile
// column of the group's M tiles.  A block-wide scan over WT threads; ends
// with a barrier.
__device__ __forceinline__ void build_cost_prefix(const int* s_offs, int G, int* s_cpref,
                                                  int* s_red, int* s_carry) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    *s_carry = 0;
    s_cpref[0] = 0;
  }
  __syncthreads();
  for (int g0 = 0; g0 < G; g0 += WT) {
    const int g = g0 + tid;
    int v = 0;
    if (g < G) {
      const int rows = s_offs[g + 1] - s_offs[g], rem = rows & (WBM - 1);
      v = (rows / WBM) * COST_FULL + last_tile_cost(rem);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(v, o, 64);
      if (lane >= o) v += n;
    }
    if (lane == 63) s_red[wv] = v;
    __syncthreads();
    int add = *s_carry;
    for (int w = 0; w < wv; ++w) add += s_red[w];
    if (g < G) s_cpref[g + 1] = add + v;
    __syncthreads();
    if (tid == WT - 1) *s_carry = add + v;
    __syncthreads();
  }
}

template <bool SWIGLU, bool GATHER, bool KEEP = false, bool BT = false>
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
  const int64_t N = args.N, ntiles = args.ntiles;
  const uint32_t K = (uint32_t)args.K;
  const int nkb = (int)(K >> 7);  // even, >= 6 (host)
  const int spt = 2 * nkb;        // steps per tile, a multiple of 4, >= 12
  const int nblk = (int)(N >> 7);
  // small copies per wave per step: 1 scale (+ 1 row-index table); the first
  // step of a K block also issues the 8 tile copies of the next block
  constexpr int NS = GATHER ? 2 : 1;

  build_group_tables<WT, WBM>(args.offs, G, s_offs, s_pref, s_red, &s_carry);
  const int64_t total = (int64_t)s_pref[G] * ntiles;
  // Tiles are numbered group by group, then in blocks of NBW N tiles (the
  // last block may be narrower), M tile by M tile, N tile last: tiles close
  // in number share weight panels (same N tile) or token rows (same M tile).
  // Blocks of 4 (32 consecutive tiles of a large group read 8 row panels and
  // 4 weight panels) time faster for the fused gate+up shapes, single N tiles
  // for the plain ones (K = 2048, N = 7168).  The workgroups of an XCD
  // (blockIdx % 8) take a contiguous range of tile numbers of equal
  // estimated cost, so that what they read together shares that XCD's L2;
  // within it workgroup j takes every (grid/8)-th tile from j on.  The cost
  // table sits in stage 1, which the first copies write only after the
  // prologue's barrier.
  constexpr int NBW = SWIGLU ? 4 : 1;
  int* s_cpref = reinterpret_cast<int*>(smem + ST_BYTES);
  build_cost_prefix(s_offs, G, s_cpref, s_red, &s_carry);
  const int64_t ctot = (int64_t)s_cpref[G] * ntiles;
  // first tile whose cost before it is at least c (total if c >= ctot)
  auto tile_at_cost = [&](int64_t c) -> int64_t {
    if (c >= ctot) return total;
    int lo = 0, hi = G - 1;  // the first group with cost past c
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)s_cpref[mid + 1] * ntiles > c) hi = mid;
      else lo = mid + 1;
    }
    // cost d into the group: N-tile block b, then (cnt - 1) rows of w full
    // tiles and a row of w last tiles (cost cl each)
    const int64_t d = c - (int64_t)s_cpref[lo] * ntiles;
    const int cg = s_cpref[lo + 1] - s_cpref[lo], cnt = s_pref[lo + 1] - s_pref[lo];
    const int cl = cg - (cnt - 1) * COST_FULL;
    const int64_t b = d / ((int64_t)NBW * cg);
    const int w = (int)min((int64_t)NBW, ntiles - NBW * b);
    const int64_t d2 = d - b * NBW * cg, dfull = (int64_t)(cnt - 1) * w * COST_FULL;
    int64_t idx = d2 <= dfull ? (d2 + COST_FULL - 1) / COST_FULL
                              : (int64_t)(cnt - 1) * w + (d2 - dfull + cl - 1) / cl;
    idx = min(idx, (int64_t)cnt * w);
    return (int64_t)s_pref[lo] * ntiles + b * NBW * cnt + idx;
  };
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3, nper = gridDim.x >> 3;
  const int64_t tlo = tile_at_cost(ctot * xcd / 8), thi = tile_at_cost(ctot * (xcd + 1) / 8);
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
    const uint32_t b = rem / (NBW * cnt), r2 = rem - b * NBW * cnt;
    const uint32_t w = (uint32_t)min((int64_t)NBW, ntiles - NBW * (int64_t)b);
    const uint32_t m = r2 / w;
    t.g = g;
    t.nt = __builtin_amdgcn_readfirstlane((int)(NBW * b + r2 - m * w));
    t.m0 = __builtin_amdgcn_readfirstlane(s_offs[g] + (int)m * WBM);
    t.m1 = __builtin_amdgcn_readfirstlane(s_offs[g + 1]);
    return t;
  };
  int gh = __builtin_amdgcn_readfirstlane(decode_tile(s_pref, s_offs, G, ntiles, L0, WBM).g);
  // weight block (of 128 columns) of the tile's column half b
  auto nblk_of = [&](const Tile& t, int b) -> int {
    return SWIGLU ? (b ? (int)(args.I >> 7) + (int)t.nt : (int)t.nt) : 2 * (int)t.nt + b;
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  // ---- copy sources of one tile.  Stage rows are 128 B with 16 B chunk c
  // of row r in slot c ^ swz(r) (conflict-free operand reads).  Wave wv
  // copies rows 32wv..32wv+31 of A and of B in 4 copies of 8 rows: copy p
  // covers rows 32wv + rb(p) + lane/8 (rb = 0, 16, 8, 24: copies 0, 1 and
  // 2, 3 share swz), lane -> LDS slot lane%8 <- global chunk
  // (lane%8) ^ swz(row).  Scales: waves 0-3 copy sA of 64 rows each, waves
  // 4-7 the two sB of the tile (the same bytes to the same place).  Gathered
  // A rows come from the tile's row-index table in LDS (buffer ord & 3),
  // clamped to A.
  struct Srcs {
    v4i rb;             // the group's B
    uint32_t va[4];     // A lane offsets of copies 0..3
    uint32_t vb[2];     // B lane offsets of copies 0 and 2 (1, 3: 16 rows further)
    uint32_t vs;        // scale lane offset
    bool a_live;        // the wave's 32 A rows reach into the tile
  };
  auto crow = [&](int p) -> int { return 32 * wv + 16 * (p & 1) + 8 * (p >> 1) + (lane >> 3); };
  // A and the scales are addressed whole (32-bit offsets: the host checks
  // the sizes); only B's base moves with the tile's group
  const uint32_t a_last = (uint32_t)(args.A_rows - 1);
  const v4i ra = load_rsrc(args.A, (uint32_t)args.A_rows * K);
  const v4i rs = wv < 4 ? load_rsrc(args.A_scale, (uint32_t)args.A_rows * (uint32_t)nkb * 4)
                        : load_rsrc(args.B_scale, (uint32_t)(G * nblk * nkb * 4));
  // source row of tile row `row` (gathered: from the table, clamped to A)
  auto a_row = [&](const Tile& t, int ord, int row) -> uint32_t {
    if (GATHER) return min((uint32_t)s_ridx[(ord & 3) * 256 + row], a_last);
    return (uint32_t)min(t.m0 + row, t.m1 - 1);
  };
  auto make_srcs = [&](const Tile& t, int ord) {
    Srcs r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int row = crow(p);
      r.va[p] = a_row(t, ord, row) * K + (uint32_t)((lane & 7) ^ swz(row)) * 16;
    }
    r.rb = load_rsrc(args.B + ((int64_t)t.g * N) * K, (uint32_t)N * K);
    r.a_live = 32 * wv < t.m1 - t.m0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (BT) {
        // W in its forward layout: stage row = contraction index within the
        // K block (this wave's rows 16wv + 4h + lane/16, and 8 further),
        // 256 output bytes per row, 16 B chunk c of row r in slot c ^ (r & 7)
        const int row = 16 * wv + 4 * h + (lane >> 4);
        r.vb[h] = (uint32_t)row * (uint32_t)N + 256u * (uint32_t)t.nt +
                  (uint32_t)(((lane & 15) ^ (row & 7)) << 4);
        continue;
      }
      const int row = crow(2 * h);
      uint32_t n;
      if (SWIGLU) n = (uint32_t)((row < 128 ? 0 : (int)args.I - 128) + 128 * (int)t.nt + row);
      else n = (uint32_t)(256 * (int)t.nt + row);
      r.vb[h] = n * K + (uint32_t)((lane & 7) ^ swz(row)) * 16;
    }
    if (wv < 4) r.vs = a_row(t, ord, 64 * wv + lane) * (uint32_t)nkb * 4;
    else if (BT) r.vs = (uint32_t)((t.g * nkb * nblk + nblk_of(t, lane == 1)) * 4);
    else r.vs = (uint32_t)((t.g * nblk + nblk_of(t, lane == 1)) * nkb * 4);
    return r;
  };
  // row-index table of a tile: slice wv & 3 (64 rows) from every wave
  auto table_src = [&](const Tile& t) -> const int32_t* {
    return args.a_row_index + min(t.m0 + 64 * (wv & 3) + lane, t.m1 - 1);
  };
  auto table_m0 = [&](int ord) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds0 + OFF_RIDX + (uint32_t)(((ord & 3) * 256 + 64 * (wv & 3)) * 4)));
  };
  auto table_copy = [&](const int32_t* src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0)
                 : "memory", "m0");
  };
  // LDS destinations: this wave's first tile-copy row, its scale slice
  const uint32_t m0_w =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + (uint32_t)(32 * wv) * 128));
  const uint32_t sc_w = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(lds0 + OFF_SC + (wv < 4 ? (uint32_t)wv * 256 : 1024u)));
  const uint32_t k16 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(16 * K));
  // BT: a K block of B is 128 rows of N bytes; copies 6, 7 are 8 rows further
  const uint32_t n128 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(128 * N));
  const uint32_t n8 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(8 * N));
  // tile copy op of K block at global offset so into stage TST: 0..3 A
  // copies, 4..7 B copies
  auto tile_op = [&](auto TST_, const Srcs& r, int op, uint32_t so) __attribute__((always_inline)) {
    constexpr int TST = decltype(TST_)::value;
    constexpr int A0 = TST * ST_BYTES, B0 = OFF_B + TST * ST_BYTES;
    // rows past the tile's end are never stored: their A copies are left out
    // (the stage keeps older bytes there)
    if (op < 4 && !r.a_live) return;
    if (BT && op >= 4) {
      // copy 4 + p: stage rows 16wv + 4p .. +3 (1 KB), from the K block's
      // 128 W rows (so / 128 = the K block)
      const uint32_t sob = (so >> 7) * n128;
      switch (op) {
        case 4: copy16<B0>(r.rb, r.vb[0], sob, m0_w); break;
        case 5: copy16<B0 + 1024>(r.rb, r.vb[1], sob, m0_w); break;
        case 6: copy16<B0 + 2048>(r.rb, r.vb[0], sob + n8, m0_w); break;
        default: copy16<B0 + 3072>(r.rb, r.vb[1], sob + n8, m0_w); break;
      }
      return;
    }
    switch (op) {
      case 0: copy16<A0>(ra, r.va[0], so, m0_w); break;
      case 1: copy16<A0 + 16 * 128>(ra, r.va[1], so, m0_w); break;
      case 2: copy16<A0 + 8 * 128>(ra, r.va[2], so, m0_w); break;
      case 3: copy16<A0 + 24 * 128>(ra, r.va[3], so, m0_w); break;
      case 4: copy16<B0>(r.rb, r.vb[0], so, m0_w); break;
      case 5: copy16<B0 + 16 * 128>(r.rb, r.vb[0], so + k16, m0_w); break;
      case 6: copy16<B0 + 8 * 128>(r.rb, r.vb[1], so, m0_w); break;
      default: copy16<B0 + 24 * 128>(r.rb, r.vb[1], so + k16, m0_w); break;
    }
  };
  // BT: the weight scales are [G, K/128, N/128] (the forward layout of W)
  const uint32_t sstride = (uint32_t)__builtin_amdgcn_readfirstlane(BT && wv >= 4 ? nblk * 4 : 4);
  auto scale_copy = [&](const Srcs& r, int kb, int gslot) __attribute__((always_inline)) {
    copy4(rs, r.vs, (uint32_t)kb * sstride, sc_w + (uint32_t)gslot * SSLOT);
  };

  // ---- prologue: table of tile 0, then its first K block and the scales
  // of its first 3 K blocks; all waited for.
  Tile tc = tile_at(gh, 0);
  const int32_t* tb_c = nullptr;
  const int32_t* tb_n = nullptr;
  uint32_t tbm_c = 0, tbm_n = 0;
  if (GATHER) {
    tb_c = table_src(tc);
    tbm_c = table_m0(0);
    table_copy(tb_c, tbm_c);
    wait_vm_lgkm0();
    barrier();
  }
  Srcs cur = make_srcs(tc, 0);
  Srcs nxt = cur;
#pragma unroll
  for (int op = 0; op < 8; ++op) tile_op(ic<0>(), cur, op, 0);
  scale_copy(cur, 0, 0);
  scale_copy(cur, 1, 1);
  scale_copy(cur, 2, 2);
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
  // 32 B K slice in step half h of a K block (chunks 4h + 2q, 4h + 2q + 1;
  // rows are multiples of 32 plus l32, so swz depends on l32 only);
  // everything else (stage, row block) is a compile-time offset.
  const int sw = swz(l32);
  uint32_t o_lo[2], o_hi[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    o_lo[h] = (uint32_t)(l32 * 128 + (((4 * h + 2 * q) ^ sw) << 4));
    o_hi[h] = (uint32_t)(l32 * 128 + (((4 * h + 2 * q + 1) ^ sw) << 4));
  }
  const uint8_t* pa = smem + wm * 64 * 128;
  const uint8_t* pb = smem + OFF_B + (SWIGLU ? wn * 64 : wn * 128) * 128;
  auto read_frag = [&](const uint8_t* lo, const uint8_t* hi, int off) -> v8i {
    const uint4 a = *reinterpret_cast<const uint4*>(lo + off);
    const uint4 b = *reinterpret_cast<const uint4*>(hi + off);
    v8i r;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    return r;
  };
  // BT: the x operand of column block j from W's forward layout by LDS
  // transpose reads.  Lane i of a 16-lane group addresses the 8 bytes at
  // stage row n0 + i/2, output byte c0 + 8 (i & 1); the read hands lane l
  // byte l % 8 of the group's chunks 2b + (l / 8) % 2, b = 0..7, i.e. the
  // column c0 + l % 16 at rows n0 .. n0 + 7.  A group covers 16 columns
  // (c0 = 128 wn + 32 j + 16 (group & 1)) and, with n0 = 64 h + 32 (group /
  // 2) + 8 r for r = 0..3, its lanes' 32 contraction bytes in the order of
  // the A operand's K bytes.  Rows n0 + b have (row & 7) = i / 2, which fixes
  // the swizzled chunk per lane and column block.
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  const __attribute__((address_space(3))) uint8_t* lds_b =
      (const __attribute__((address_space(3))) uint8_t*)smem + OFF_B;
  uint32_t o_tr[4];
  {
    const int grp = lane >> 4, li = lane & 15;
    const int base = (32 * (grp >> 1) + (li >> 1)) * 256 + 8 * (li & 1) + 128 * wn;
#pragma unroll
    for (int j = 0; j < 4; ++j) o_tr[j] = (uint32_t)(base + (((2 * j + (grp & 1)) ^ (li >> 1)) << 4));
  }
  // B stage row offset (from the wave's base row) of column block j
  auto b_roff = [&](int j) -> int { return SWIGLU ? (j < 2 ? 32 * j : 128 + 32 * (j - 2)) : 32 * j; };
  auto half_of = [&](int j) -> int { return SWIGLU ? (j >= 2) : wn; };

  int gh_n = gh;  // hint for decoding the next tile
  Tile tn = tc;
  v8i a[2], b[4];  // MFMA operands of the current step (A rows, B rows)
  // operands of step half HH of the K block in stage STG
  auto read_ops = [&](auto STG_, auto HH_) __attribute__((always_inline)) {
    constexpr int STG = decltype(STG_)::value, HH = decltype(HH_)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = read_frag(pa + o_lo[HH], pa + o_hi[HH], STG * ST_BYTES + i * 32 * 128);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (BT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_v2i*)(lds_b + STG * ST_BYTES + (64 * HH + 8 * r) * 256 + o_tr[j]));
          b[j][2 * r] = t[0];
          b[j][2 * r + 1] = t[1];
        }
      } else {
        b[j] = read_frag(pb + o_lo[HH], pb + o_hi[HH], STG * ST_BYTES + b_roff(j) * 128);
      }
  };
  read_ops(ic<0>(), ic<0>());

  for (int ord = 0; ord < my_n; ++ord) {
    const bool has_next = ord + 1 < my_n;
    const bool wvalid = tc.m0 + 64 * wm < tc.m1;
    const int gbase = ord * nkb;  // global K-block index of this tile's kb 0

    // One step k = k4 + U of this tile (stage U: tiles start at a multiple
    // of 4 steps; K block k4/2 + U/2).  Phase PH: 0 the first 4 steps (k4 =
    // 0), 1 the interior (4 <= k4 < spt - 8), 2 and 3 the last 8 (k4 = spt -
    // 8, spt - 4; spt >= 12).  Every test below is decided by U and PH
    // except the first step's wait for the previous epilogue's stores.
    // After the last tile the copies still run (onto the last tile's own
    // sources), so every K block issues the same copies.
    auto step = [&](auto U_, auto PH_, int k4) __attribute__((always_inline)) {
      constexpr int U = decltype(U_)::value;
      constexpr int PH = decltype(PH_)::value;
      const int k = k4 + U;
      // second step of a K block: everyone is past the first (whose ratios
      // it uses); the first step of a K block synchronises at the end of the
      // block before
      if ((U & 1) == 1) {
        wait_lgkm0();
        barrier();
      }

      // ---- next tile: decode (its table is copied from step spt-8 on) and
      // copy sources (at step spt-5, when that table has landed)
      if (PH == 2 && U == (GATHER ? 0 : 3)) {
        tn = has_next ? tile_at(gh_n, ord + 1) : tc;
        if (GATHER) {
          tb_n = table_src(tn);
          tbm_n = table_m0(ord + 1);
        }
      }
      if (PH == 2 && U == 3) nxt = make_srcs(tn, ord + 1);
      // ---- scales of the K block of step k+5 (re-copied: same data); in
      // the last 5 steps, the next tile's first blocks
      {
        constexpr bool NEXT = PH == 3 || (PH == 2 && U == 3);
        const int kb5 = (k + 5) >> 1;
        const int gslot = (gbase + kb5) & 3;
        if (NEXT) scale_copy(nxt, kb5 - nkb, gslot);
        else scale_copy(cur, kb5, gslot);
      }
      // ---- the current or next tile's row-index table (re-copied)
      if (GATHER) {
        if (PH >= 2) table_copy(tb_n, tbm_n);
        else table_copy(tb_c, tbm_c);
      }
      // ---- the first step of K block kb copies block kb+1 into the other
      // stage, between its MFMAs (the last block: the next tile's block 0)
      constexpr bool T_COPY = (U & 1) == 0;
      constexpr bool T_NEXT = PH == 3 && U == 2;
      constexpr int ST = U >> 1;              // stage of step k (k4 / 2 is even)
      constexpr int H = U & 1;                // half of the K block
      constexpr int TST = ST ^ 1;             // stage of block kb+1
      const uint32_t so = (uint32_t)((T_NEXT ? 0 : (k >> 1) + 1) * 128);
      auto copies = [&](int op) __attribute__((always_inline)) {
        if (!T_COPY) return;
        if (T_NEXT) tile_op(ic<TST>(), nxt, op, so);
        else tile_op(ic<TST>(), cur, op, so);
      };

      const int kb = (k4 >> 1) + (U >> 1);
      // rescale by S_kb-1 / S_kb in two halves: column blocks 2, 3 in the
      // first step of K block kb, blocks 0, 1 in the step before; each step
      // carries half of the multiplies.  None before K block 1; none after
      // the last block.
      constexpr bool RESC_NOW = (U & 1) == 0 && !(PH == 0 && U == 0);
      constexpr bool RESC_NEXT = (U & 1) == 1 && !(PH == 3 && U == 3);
      // ratios S_kb / S_kb+1 after a K block's first step, but the last
      constexpr bool RATIO = (U & 1) == 0 && !(PH == 3 && U == 2);
      // ratios S_kb / S_kb+1 for the next K block of this tile, one (row,
      // column half) per thread: scales read at the start of a K block's
      // first step, the quotient stored between its MFMAs (read from the
      // next step on, after its barrier)
      float rsc[4];
      const int rrow = tid & 255, rb = tid >> 8;
      auto ratio_load = [&]() __attribute__((always_inline)) {
        const float* sc0 = s_sc + ((gbase + kb) & 3) * (SSLOT / 4);
        const float* sc1 = s_sc + ((gbase + kb + 1) & 3) * (SSLOT / 4);
        rsc[0] = sc0[rrow]; rsc[1] = sc0[256 + rb];
        rsc[2] = sc1[rrow]; rsc[3] = sc1[256 + rb];
      };
      auto ratio_store = [&]() __attribute__((always_inline)) {
        s_r[((kb + 1) & 1) * 512 + rb * 256 + rrow] = (rsc[0] * rsc[1]) / (rsc[2] * rsc[3]);
      };
      if (wvalid) {
        // this step's operands are in registers: a K block's first-step
        // operands were read at the end of the block before (after its
        // wait and barrier), its second step's at the end of its first step
        // (same stage), so their LDS latency hides behind MFMAs
        if (RATIO) ratio_load();
        // the ratio of a (token row, column half) pair: one value per lane
        // and row block
        auto load_ratios = [&](float* rr, int kbr, int hb) __attribute__((always_inline)) {
          const float* rsh = s_r + (kbr & 1) * 512 + hb * 256 + wm * 64 + l32;
          rr[0] = rsh[0];
          rr[1] = rsh[32];
        };
        auto rescale = [&](int i, int j, float r_) __attribute__((always_inline)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= r_;
        };
        float r_now[2], r_next[2];
        if (RESC_NOW) load_ratios(r_now, kb, SWIGLU ? 1 : wn);
        if (RESC_NEXT) load_ratios(r_next, kb + 1, SWIGLU ? 0 : wn);
        // MFMA s = (block j = s/2, row block i = s%2); after each of the
        // first four, a quarter of blocks 2, 3's rescale (before their own
        // MFMAs), after each of the last four, a quarter of blocks 0, 1's
        // rescale for the next K block (after theirs): 16 multiplies between
        // consecutive MFMAs, which the other wave's MFMAs cover
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int j = s >> 1, i = s & 1;
          acc[i][j] = mfma32(b[j], a[i], acc[i][j]);
          copies(s);
          if (RESC_NOW && s < 4) rescale(s & 1, 2 + (s >> 1), r_now[s & 1]);
          if (RESC_NEXT && s >= 4) rescale(s & 1, (s - 4) >> 1, r_next[s & 1]);
          if (RATIO && s == 5) ratio_store();
          __builtin_amdgcn_sched_barrier(0);  // keep this order (the scheduler would group)
        }
        if (H == 0) read_ops(ic<ST>(), ic<1>());
      } else {
#pragma unroll
        for (int op = 0; op < 8; ++op) copies(op);
        if (RATIO) {
          ratio_load();
          ratio_store();
        }
      }
      // end of a K block: the next block's copies (issued in this block's
      // first step) are done, only this step's small copies may still fly
      // (in a tile's first block: everything, as the last epilogue's stores
      // count too); then everyone is past this block (its stage is free) and
      // the next block's first-step operands are read (the next tile's block
      // 0 after a tile's last block; every wave, valid in the next tile or
      // not)
      if ((U & 1) == 1) {
        if (PH == 0 && U == 1) wait_vm_lgkm0();
        else wait_vmcnt_lgkm0<NS>();
        barrier();
        read_ops(ic<(U == 1 ? 1 : 0)>(), ic<0>());
      }
    };
    step(ic<0>(), ic<0>(), 0);
    step(ic<1>(), ic<0>(), 0);
    step(ic<2>(), ic<0>(), 0);
    step(ic<3>(), ic<0>(), 0);
    for (int k4 = 4; k4 < spt - 8; k4 += 4) {
      step(ic<0>(), ic<1>(), k4);
      step(ic<1>(), ic<1>(), k4);
      step(ic<2>(), ic<1>(), k4);
      step(ic<3>(), ic<1>(), k4);
    }
    step(ic<0>(), ic<2>(), spt - 8);
    step(ic<1>(), ic<2>(), spt - 8);
    step(ic<2>(), ic<2>(), spt - 8);
    step(ic<3>(), ic<2>(), spt - 8);
    step(ic<0>(), ic<3>(), spt - 4);
    step(ic<1>(), ic<3>(), spt - 4);
    step(ic<2>(), ic<3>(), spt - 4);
    step(ic<3>(), ic<3>(), spt - 4);

    // ---- epilogue of tile ord: result = acc * S_last.  Lane (q, l32) of
    // wave (wm, wn) holds tile row wm*64 + 32i + l32 of row block i and, in
    // column block j, the columns 8g + 4q + (0..3) for g = 0..3.
    const Tile t = tc;
    const float* scl = s_sc + ((gbase + nkb - 1) & 3) * (SSLOT / 4);
    if (wvalid) {
      const float sb[2] = {scl[256], scl[257]};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float sa = scl[wm * 64 + 32 * i + l32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float S = sa * sb[half_of(j)];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] *= S;
        }
      }
    }
    if (!SWIGLU) {
      // bf16 (round to nearest even), staged through LDS so that each store
      // writes whole 128 B rows: per half of its columns (j = 2c, 2c+1) a
      // wave writes its 64 rows x 64 columns into its own 8 KB of the
      // tile's free K-block stage (stage 1: the last K block's, all of whose
      // reads ended at the last step's barrier; 16 B chunks XOR-swizzled by
      // row), reads them back 8 rows x 128 B per instruction and stores them.
      // Only the wave itself touches its region; the barrier after the
      // epilogue keeps the next tile's copies into stage 1 behind it.
      if (wvalid) {
        const uint32_t rowb = (uint32_t)N * 2;
        const __amdgpu_buffer_rsrc_t rs =
            out_rsrc(args.C + (int64_t)t.m0 * N, (uint32_t)min(t.m1 - t.m0, WBM) * rowb);
        uint8_t* reg = smem + (wv < 4 ? ST_BYTES + wv * 8192 : OFF_B + ST_BYTES + (wv - 4) * 8192);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int row = 32 * i + l32;  // in the wave's 64
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const v16f& v = acc[i][2 * c + jj];
                typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                const v2u w = {f32x2_to_bf16x2(v[4 * g], v[4 * g + 1]),
                               f32x2_to_bf16x2(v[4 * g + 2], v[4 * g + 3])};
                const int chunk = (4 * jj + g) ^ (row & 7);
                *reinterpret_cast<v2u*>(reg + row * 128 + chunk * 16 + q * 8) = w;
              }
          }
          wait_lgkm0();
          const int vb = (wm * 64 + (lane >> 3)) * (int)rowb +
                         (int)(256 * t.nt + wn * 128 + 64 * c + 8 * (lane & 7)) * 2;
#pragma unroll
          for (int r8 = 0; r8 < 8; ++r8) {
            const int row = 8 * r8 + (lane >> 3);
            const uint4 d = *reinterpret_cast<const uint4*>(reg + row * 128 + (((lane & 7) ^ (row & 7)) << 4));
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u w = {d.x, d.y, d.z, d.w};
            __builtin_amdgcn_raw_buffer_store_b128(w, rs, vb, 8 * r8 * (int)rowb, 0);
          }
          wait_lgkm0();
        }
      }
    } else {
      // KEEP: the bf16 gate/up sums too, staged like the plain epilogue (a
      // wave's 64 rows x 64 columns per half, in its own 8 KB of stage 1;
      // every wave's reads are done before the barrier below, after which
      // the codes reuse that memory).  Half c = 0 holds gate columns
      // 128 nt + 64 wn + 32 jj + 8 g + 4 q (+0..3) of blocks j = jj, half
      // c = 1 the up columns I + the same, of blocks j = 2 + jj.
      if (KEEP && wvalid) {
        const int I2 = 2 * (int)args.I;
        const uint32_t rowb = (uint32_t)I2 * 2;
        const __amdgpu_buffer_rsrc_t rs =
            out_rsrc(args.GU + (int64_t)t.m0 * I2, (uint32_t)min(t.m1 - t.m0, WBM) * rowb);
        uint8_t* reg = smem + (wv < 4 ? ST_BYTES + wv * 8192 : OFF_B + ST_BYTES + (wv - 4) * 8192);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int row = 32 * i + l32;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const v16f& v = acc[i][2 * c + jj];
                typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                const v2u w = {f32x2_to_bf16x2(v[4 * g], v[4 * g + 1]),
                               f32x2_to_bf16x2(v[4 * g + 2], v[4 * g + 3])};
                const int chunk = (4 * jj + g) ^ (row & 7);
                *reinterpret_cast<v2u*>(reg + row * 128 + chunk * 16 + q * 8) = w;
              }
          }
          wait_lgkm0();
          const int vb = (wm * 64 + (lane >> 3)) * (int)rowb +
                         (c * (int)args.I + (int)(128 * t.nt) + 64 * wn + 8 * (lane & 7)) * 2;
#pragma unroll
          for (int r8 = 0; r8 < 8; ++r8) {
            const int row = 8 * r8 + (lane >> 3);
            const uint4 d = *reinterpret_cast<const uint4*>(reg + row * 128 + (((lane & 7) ^ (row & 7)) << 4));
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u w = {d.x, d.y, d.z, d.w};
            __builtin_amdgcn_raw_buffer_store_b128(w, rs, vb, 8 * r8 * (int)rowb, 0);
          }
          wait_lgkm0();
        }
      }
      // the row pair's (wm) 64 rows x 128 B of codes, staged in the tile's
      // free K-block stage (A part of stage 1) for whole-row stores
      uint8_t* hreg = smem + ST_BYTES + wm * 8192;
      // h = silu(g) * u: gate block j pairs with up block j + 2.  A row's 128
      // h columns of this N tile: 32 in each lane of the pair (q = 0, 1) of
      // both column waves; the row maximum meets over the pair by a lane
      // exchange and over the two waves in LDS.
      float inv[2] = {1.f, 1.f};
      if (wvalid) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float g = acc[i][j][r], u = acc[i][j + 2][r];
              const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
              const float h = g * __builtin_amdgcn_rcpf(1.0f + e) * u;
              acc[i][j][r] = h;
              m = fmaxf(m, fabsf(h));
            }
          m = fmaxf(m, __shfl_xor(m, 32, 64));
          s_amax[(wm * 64 + 32 * i + l32) * 2 + wn] = m;  // both lanes of the pair: same value
        }
      }
      wait_lgkm0();
      barrier();
      if (wvalid) {
        // hb passes through an empty asm so that the per-row scale offsets
        // below are computed here, not kept live across the K loop (they
        // had cost a spilled VGPR whose reload waited for every copy)
        const int I = (int)args.I;
        int hb = I >> 7;
        asm volatile("" : "+s"(hb));
        const uint32_t rows = (uint32_t)min(t.m1 - t.m0, WBM);
        const __amdgpu_buffer_rsrc_t rsc = out_rsrc(args.Hs + (int64_t)t.m0 * hb, rows * hb * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int trow = wm * 64 + 32 * i + l32;
          const float amax = fmaxf(s_amax[trow * 2], s_amax[trow * 2 + 1]);
          const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
          inv[i] = 1.0f / sc;
          if (wn == 0 && q == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsc, (trow * hb + (int)t.nt) * 4, 0, 0);
          // codes into the pair's 64 rows x 128 B of LDS (16 B chunks
          // swizzled by row): columns wn*64 + 32j + 8g + 4q, 4 per dword
          const int row = 32 * i + l32;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const v16f& h = acc[i][j];
              const int chunk = (4 * wn + 2 * j + (g >> 1)) ^ (row & 7);
              *reinterpret_cast<uint32_t*>(hreg + row * 128 + chunk * 16 + 8 * (g & 1) + 4 * q) =
                  f32x4_to_e4m3x4(h[4 * g] * inv[i], h[4 * g + 1] * inv[i], h[4 * g + 2] * inv[i],
                                  h[4 * g + 3] * inv[i]);
            }
        }
      }
      wait_lgkm0();
      barrier();
      // whole 128 B rows: wave wn stores rows 32wn..32wn+31 of its pair's 64
      if (wvalid) {
        const int I = (int)args.I;
        const uint32_t rows = (uint32_t)min(t.m1 - t.m0, WBM);
        const __amdgpu_buffer_rsrc_t rq = out_rsrc(args.Hq + (int64_t)t.m0 * I, rows * I);
        const int vq = (wm * 64 + 32 * wn + (lane >> 3)) * I + (int)(128 * t.nt) + 16 * (lane & 7);
#pragma unroll
        for (int r8 = 0; r8 < 4; ++r8) {
          const int row = 32 * wn + 8 * r8 + (lane >> 3);
          const uint4 d = *reinterpret_cast<const uint4*>(hreg + row * 128 + (((lane & 7) ^ (row & 7)) << 4));
          typedef uint32_t v4u __attribute__((ext_vector_type(4)));
          const v4u w = {d.x, d.y, d.z, d.w};
          __builtin_amdgcn_raw_buffer_store_b128(w, rq, vq, 8 * r8 * I, 0);
        }
      }
    }
    // the next tile's copies into stage 1 wait for every wave's epilogue
    barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // (the epilogue's stores count in vmcnt and may finish out of order:
    // the next tile's first step waits for everything)
    tc = tn;
    cur = nxt;
    tb_c = tb_n;
    tbm_c = tbm_n;
  }
  wait_vm_lgkm0();  // copies issued past the last tile land before the LDS is released
}

}  // namespace

int launch_wide(const GemmArgs& a, bool swiglu, hipStream_t st) {
  const int grid = std::max(8, (num_cus() / 8) * 8);
  if (swiglu && a.GU) {
    if (a.a_row_index) wide_gemm_kernel<true, true, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
    else wide_gemm_kernel<true, false, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
  } else if (swiglu) {
    if (a.a_row_index) wide_gemm_kernel<true, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
    else wide_gemm_kernel<true, false><<<dim3(grid), dim3(WT), 0, st>>>(a);
  } else {
    if (a.a_row_index) wide_gemm_kernel<false, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
    else wide_gemm_kernel<false, false><<<dim3(grid), dim3(WT), 0, st>>>(a);
  }
  return MOE_OK;
}

int launch_wide_bt(const GemmArgs& a, hipStream_t st) {
  const int grid = std::max(8, (num_cus() / 8) * 8);
  wide_gemm_kernel<false, false, false, true><<<dim3(grid), dim3(WT), 0, st>>>(a);
  return MOE_OK;
}

}  // namespace gemm
}  // namespace moe
