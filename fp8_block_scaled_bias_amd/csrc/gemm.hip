// Block-scaled FP8 grouped GEMM for small and medium groups (row tiles of
// 32, 64 or 128), with an optional fused SwiGLU + 1x128 requantisation
// epilogue, and the host entry points that choose between it and the
// 256x256-tile kernel of gemm_wide.hip.
//
// Method: news.qq.com/rain/a/20241229A05OQF00, section FP8 低精度训练 -
// activations carry one fp32 scale per 1x128 tile and weights one per
// 128x128 block (细粒度量化), and MMA partial results are accumulated in FP32
// at a fixed K interval (提高累加精度).
//
// gfx950 design
//  * One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-wide K block of
//    a 16x16 output tile, so its result P is that block's partial sum.  It is
//    issued with a zero accumulator and promoted at once:
//        acc += (sA[row, kb] * sB[nblk, kb]) * P      (one FMA per output)
//    The MFMA's own 128-term sum is not fp32-exact (the hardware's
//    limited-precision dot product, the effect the 128-element promotion
//    interval bounds); everything after it is fp32.
//  * Workgroup tile BM x 256 (4 waves), K step 128.  Tiles of A (BM x 128 B),
//    B (256 x 128 B) and A's scales (one fp32 per row) are copied global ->
//    LDS with global_load_lds_dwordx4 / _dword (no VGPR staging) into a ring
//    of STAGES buffers, so STAGES-1 K blocks are in flight while one is
//    consumed.  The copies are issued from inline asm and their completion is
//    tracked with explicit vmcnt waits plus a workgroup barrier per K block.
//  * Persistent: one workgroup per CU walks an XCD-local range of the tile
//    list (see decode_tile); rows past a group's end are clamped on load and
//    masked on store (an output row depends only on its own A row).
//  * Epilogues: bf16 (round to nearest even), four lanes' columns packed into
//    one 8-byte store; or SwiGLU: the 256 columns are 128 gate + 128 up
//    columns of the same h block, h = silu(g) * u is formed in fp32 from the
//    fp32 accumulators (g and u are never stored) and quantised 1x128 to E4M3.
#include "gemm_common.h"

namespace moe {
namespace gemm {
namespace {

constexpr int GM_THREADS = 256;
constexpr int BN = 256;

template <int BM, int WAVES_M, int STAGES, bool SWIGLU, bool GATHER, bool EXACT = false>
struct Cfg {
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WTM = BM / WAVES_M;
  static constexpr int WTN = BN / WAVES_N;  // B tile rows a wave multiplies
  static constexpr int SI = WTM / 16;
  static constexpr int SJ = WTN / 16;
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BN * 128;
  static constexpr int S_BYTES = 256 * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int A_LOADS = BM / 32;  // dwordx4 copies per wave per step
  static constexpr int B_LOADS = 8;
  static constexpr int LOADS = A_LOADS + B_LOADS + 1 + (GATHER ? 1 : 0);
  static constexpr int OFF_PREF = STAGES * STAGE;            // int [MAXG + 1]
  static constexpr int OFF_OFFS = OFF_PREF + (MAXG + 1) * 4;  // int [MAXG + 1]
  static constexpr int OFF_RIDX = OFF_OFFS + (MAXG + 1) * 4;  // int [2][256]
  static constexpr int OFF_AMAX = OFF_RIDX + 2 * 256 * 4;     // float [BM][WAVES_N]
  static constexpr int LDS = OFF_AMAX + (SWIGLU ? BM * WAVES_N * 4 : 0);
  static_assert(WTN <= 128 || SWIGLU, "a wave's columns must lie in one 128-column block");
  static_assert(BM <= 128, "scale slots BM, BM+1 carry the weight scales");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Persistent kernel: one workgroup per CU walks its share of the tiles
// (XCD-local, see decode_tile).  The copies of K block kb of the current or
// a later tile ("steps") are issued STAGES-1 steps ahead of the step being
// multiplied, across tile boundaries, so a tile's first K blocks load while
// the previous tile finishes.  With GATHER, the A row indices of the next
// tile are copied into LDS one tile ahead (every step of a tile repeats that
// copy, so the table a new tile reads was written by a copy that has already
// been waited for).
template <int BM, int WAVES_M, int STAGES, bool SWIGLU, bool GATHER, bool EXACT, bool BT = false>
__global__ __launch_bounds__(GM_THREADS, 1) void grouped_gemm_kernel(GemmArgs args) {
  static_assert(!BT || (!SWIGLU && !GATHER && !EXACT), "BT: plain epilogue, dense A rows");
  using C_ = Cfg<BM, WAVES_M, STAGES, SWIGLU, GATHER, EXACT>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C_::LDS];
  __shared__ int s_red[4];
  __shared__ int s_carry;
  int* s_pref = reinterpret_cast<int*>(smem + C_::OFF_PREF);
  int* s_offs = reinterpret_cast<int*>(smem + C_::OFF_OFFS);
  int* s_ridx = reinterpret_cast<int*>(smem + C_::OFF_RIDX);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / C_::WAVES_N, wn = wv % C_::WAVES_N;
  const int G = args.G;
  const int64_t K = args.K, N = args.N, ntiles = args.ntiles;
  const int64_t nkb = K >> 7;

  // ---- group tables: offsets and exclusive prefix of M tiles per group ----
  build_group_tables<GM_THREADS, BM>(args.offs, G, s_offs, s_pref, s_red, &s_carry);
  const int64_t total = (int64_t)s_pref[G] * ntiles;
  // this workgroup's tiles: XCD x owns ids [x*chunk, (x+1)*chunk); its
  // workgroups (blocks x, x+8, ...) take every (gridDim/8)-th of them.  The
  // exact-sum launches (weight-stream bound, tiles of different cost: a
  // group's 16-row blocks past its end skip their instructions) stride over
  // the whole list instead, so no XCD holds all of a large group's tiles.
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const int nper = EXACT ? (int)gridDim.x : (int)(gridDim.x >> 3);
  const int64_t chunk = (total + 7) >> 3;
  const int64_t tlo = EXACT ? 0 : xcd * chunk, thi = EXACT ? total : min(total, tlo + chunk);
  const int64_t L0 = EXACT ? (int64_t)blockIdx.x : tlo + jw;
  if (L0 >= thi) return;
  const int64_t my_n = (thi - L0 + nper - 1) / nper;
  const int64_t nsteps = my_n * nkb;
  // exact-sum launches: the tiles of more than 16 rows cost several times a
  // 16-row one; in the MoE layer they are the last group's (the shared
  // expert's rows follow the routed experts').  The strided list is rotated
  // so that group's tiles sit at positions [rem, rem + n_last), rem = total
  // mod grid: the workgroups taking them are not those that also take a tile
  // of the last, partial round.
  const int64_t n_last = (int64_t)(s_pref[G] - s_pref[G - 1]) * ntiles;
  const int64_t rot =
      EXACT ? (total - ((total % (int64_t)gridDim.x) + n_last) % total) % total : 0;

  auto tile_of = [&](int64_t ord) {
    int64_t Lg = L0 + ord * nper;
    if (EXACT) Lg = (Lg + rot) % total;
    Tile t = decode_tile(s_pref, s_offs, G, ntiles, Lg, BM);
    t.g = __builtin_amdgcn_readfirstlane(t.g);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.m1 = __builtin_amdgcn_readfirstlane(t.m1);
    t.nt = __builtin_amdgcn_readfirstlane((int)t.nt);
    return t;
  };

  // ---- issue side: per-lane copy sources of the tile being issued ----
  // copy instruction q covers tile rows 8q..8q+7: lane -> row 8q + lane/8,
  // LDS slot lane%8, so it fetches global chunk (lane%8) ^ swz(row) with
  // swz(row) = (lane/8) ^ (q & 1).
  const int chunk0 = (lane & 7) ^ (lane >> 3);
  const int chunk1 = chunk0 ^ 1;
  const uint8_t* a_src[C_::A_LOADS];
  const uint8_t* b_src0 = nullptr;
  const uint8_t* b_src1 = nullptr;
  bool b_tail = false;
  const float* s_src = nullptr;
  int s_kstride = 1;  // scale elements between consecutive K blocks
  const int32_t* r_src = nullptr;  // row-index copy source (next tile)

  auto row_src = [&](const Tile& t, int64_t ord, int row) -> int64_t {
    if (GATHER) return (int64_t)min((uint32_t)s_ridx[(ord & 1) * 256 + row], (uint32_t)(args.A_rows - 1));
    return (int64_t)min(t.m0 + row, t.m1 - 1);
  };
  auto setup_issue = [&](int64_t ord) {
    const Tile t = tile_of(ord);
#pragma unroll
    for (int qi = 0; qi < C_::A_LOADS; ++qi) {
      const int q = wv * C_::A_LOADS + qi;
      const int row = 8 * q + (lane >> 3);
      a_src[qi] = args.A + row_src(t, ord, row) * K + ((q & 1) ? chunk1 : chunk0) * 16;
    }
    if (BT) {
      // W [K, N] as stored: stage row = contraction index in the K block,
      // 256 output bytes per row, chunk c of row r in slot c ^ (r & 7).
      // Copy qi covers rows 32wv + 4qi + lane/16 (slot lane%16); its source
      // chunk depends on qi & 1 only.  A last tile of 128 columns (N not a
      // multiple of 256) re-reads its valid chunks for the upper half.
      const bool half = 256 * t.nt + 256 > N;  // wave-uniform
      const uint8_t* w = args.B + (int64_t)t.g * K * N + 256 * t.nt;
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int row = 32 * wv + 4 * o + (lane >> 4);
        int c = (lane & 15) ^ (row & 7);
        if (half) c &= 7;
        (o ? b_src1 : b_src0) = w + (int64_t)row * N + c * 16;
      }
    } else {
      int64_t brow0;
      if (SWIGLU) brow0 = ((wv < 2) ? 0 : args.I) + 128 * t.nt + 64 * (wv & 1) + (lane >> 3);
      else brow0 = 256 * t.nt + 64 * wv + (lane >> 3);
      const uint8_t* b_row = args.B + ((int64_t)t.g * N + min<int64_t>(brow0, N - 1)) * K;
      b_src0 = b_row + chunk0 * 16;
      b_src1 = b_row + chunk1 * 16;
      b_tail = (brow0 - (lane >> 3)) + 64 > N;  // wave-uniform
    }
    const int srow = 64 * wv + lane;
    if (srow < BM) {
      s_src = args.A_scale + row_src(t, ord, srow) * nkb;
    } else {
      const int b = srow & 1;
      const int64_t nb = SWIGLU ? (b ? (args.I >> 7) + t.nt : t.nt)
                                : min<int64_t>(2 * t.nt + b, (N >> 7) - 1);
      if (BT) {
        s_src = args.B_scale + (int64_t)t.g * nkb * (N >> 7) + nb;  // [G, K/128, N/128]
        s_kstride = (int)(N >> 7);
      } else {
        s_src = args.B_scale + ((int64_t)t.g * (N >> 7) + nb) * nkb;
      }
    }
    if (GATHER) {
      const Tile tn = (ord + 1 < my_n) ? tile_of(ord + 1) : t;
      r_src = args.a_row_index + min(tn.m0 + min(64 * wv + lane, BM - 1), tn.m1 - 1);
    }
  };

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int nkb32 = (int)nkb;
  const int64_t K8 = 8 * K;
  const int64_t N8 = 8 * N, N128 = 128 * N;  // BT: 8 W rows, one K block of W rows
  // issue position (tile ordinal, K block, ring slot), advanced per step
  int iss_ord = 0, iss_kb = 0, iss_slot = 0;
  // One step's copies, split so they can be spread over the MFMA loop:
  // issue_begin() sets up the step (new tile: per-lane sources), issue_op(k)
  // issues copy k of LOADS, issue_end() advances the issue position.  A wave
  // that issues into a saturated memory pipeline stalls; spread between
  // MFMAs, those stalls overlap the matrix pipe's work.
  uint32_t iss_st = 0;
  int64_t iss_ko = 0;
  auto issue_begin = [&]() {
    if (iss_kb == 0) setup_issue(iss_ord);
    iss_st = lds0 + (uint32_t)iss_slot * C_::STAGE;
    iss_ko = (int64_t)iss_kb * 128;
  };
  auto issue_op = [&](int k) {
    if (k < C_::A_LOADS) {
      dma16(a_src[k] + iss_ko, iss_st + (wv * C_::A_LOADS + k) * 1024);
    } else if (k < C_::A_LOADS + C_::B_LOADS) {
      const int qi = k - C_::A_LOADS;
      if (BT)
        dma16(((qi & 1) ? b_src1 : b_src0) + (qi >> 1) * N8 + (int64_t)iss_kb * N128,
              iss_st + C_::A_BYTES + (wv * 8 + qi) * 1024);
      else
        dma16(((qi & 1) ? b_src1 : b_src0) + (b_tail ? 0 : qi * K8) + iss_ko,
              iss_st + C_::A_BYTES + (wv * 8 + qi) * 1024);
    } else if (k == C_::A_LOADS + C_::B_LOADS) {
      dma4(s_src + iss_kb * s_kstride, iss_st + C_::A_BYTES + C_::B_BYTES + wv * 256);
    } else {
      dma4(r_src, lds0 + C_::OFF_RIDX + (uint32_t)(((iss_ord + 1) & 1) * 1024 + wv * 256));
    }
  };
  auto issue_end = [&]() {
    if (++iss_kb == nkb32) {
      iss_kb = 0;
      ++iss_ord;
    }
    if (++iss_slot == STAGES) iss_slot = 0;
  };
  auto issue_step = [&]() {
    issue_begin();
#pragma unroll
    for (int k = 0; k < C_::LOADS; ++k) issue_op(k);
    issue_end();
  };

  // ---- prologue: row indices of the first tile, then STAGES-1 steps ----
  if (GATHER) {
    const Tile t0 = tile_of(0);
    dma4(args.a_row_index + min(t0.m0 + min(64 * wv + lane, BM - 1), t0.m1 - 1),
         lds0 + C_::OFF_RIDX + wv * 256);
    wait_vmcnt<0>();
    barrier();
  }
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < nsteps) {
      if (GATHER && iss_kb == 0 && iss_ord > 0) {
        // short K: this tile's row-index table was copied by a step issued
        // just before; drain before reading it
        wait_vmcnt<0>();
        barrier();
      }
      issue_step();
    }
  }

  v4f acc[C_::SI][C_::SJ];
#pragma unroll
  for (int i = 0; i < C_::SI; ++i)
#pragma unroll
    for (int j = 0; j < C_::SJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int h = lane >> 4;
  constexpr int WHN = 128 / C_::WAVES_N;  // SwiGLU: h columns per wave
  constexpr int SJH = C_::SJ / 2;
  // B tile row of this lane for column subtile j
  auto b_row_of = [&](int j) -> int {
    if (SWIGLU) return (j < SJH ? wn * WHN + 16 * j : 128 + wn * WHN + 16 * (j - SJH)) + (lane & 15);
    return wn * C_::WTN + 16 * j + (lane & 15);
  };
  // BT: column subtile j by LDS transpose reads.  Lane i of each 16-lane
  // group addresses the 8 bytes at row 32 (lane/16) + 8r + i/2, output byte
  // 16 chunk + 8 (i & 1); lane l receives byte l % 8 of the group's chunks
  // 2b + (l / 8) % 2, i.e. column 16 chunk + l % 16 at the 8 rows from
  // 32 (lane/16) + 8r: its 32 contraction bytes over r = 0..3, in the order
  // of the A operand's K bytes.  (row & 7) = i / 2 fixes the swizzled slot.
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  const int tli = lane & 15;
  const uint32_t bt_lane = (uint32_t)((32 * (lane >> 4) + (tli >> 1)) * 256 + 8 * (tli & 1));
  auto b_frag = [&](const uint8_t* tB, int j) -> v8i {
    if (!BT) return lds_frag(tB, b_row_of(j), h);
    const int chunk = (wn * C_::WTN + 16 * j) >> 4;
    const __attribute__((address_space(3))) uint8_t* p =
        (const __attribute__((address_space(3))) uint8_t*)tB + bt_lane + ((chunk ^ (tli >> 1)) << 4);
    v8i x;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p + r * 8 * 256));
      x[2 * r] = t[0];
      x[2 * r + 1] = t[1];
    }
    return x;
  };

  const int nsteps32 = (int)nsteps;
  int c_ord = 0, c_kb = 0, slot = 0;  // consume position
  int c_rows = 0;                     // rows of the tile being consumed
  for (int c = 0; c < nsteps32; ++c) {
    if (c_kb == 0) {
      const Tile tc = tile_of(c_ord);
      c_rows = __builtin_amdgcn_readfirstlane(tc.m1 - tc.m0);
    }
    const int after = min(STAGES - 2, nsteps32 - 1 - c);
    if (STAGES >= 4 && after >= 2) wait_vmcnt<(STAGES >= 4 ? 2 : 0) * C_::LOADS>();
    else if (after >= 1) wait_vmcnt<C_::LOADS>();
    else wait_vmcnt<0>();
    barrier();
    const bool do_issue = c + STAGES - 1 < nsteps32;
    if (do_issue) {
      if (GATHER && nkb32 < STAGES - 1 && iss_kb == 0) {
        // short K: the last copy of the next tile's row indices may still be
        // in flight; drain before reading the table
        wait_vmcnt<0>();
        barrier();
      }
      issue_begin();
    }

    const uint8_t* tA = smem + slot * C_::STAGE;
    const uint8_t* tB = tA + C_::A_BYTES;
    const float* tS = reinterpret_cast<const float*>(tB + C_::B_BYTES);
    float sc0[C_::SI][4], sc1[C_::SI][4];  // sc1: SwiGLU up half
    {
      const float sb0 = SWIGLU ? tS[BM] : tS[BM + ((wn * C_::WTN) >> 7)];
      const float sb1 = tS[BM + 1];
#pragma unroll
      for (int i = 0; i < C_::SI; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(tS + wm * C_::WTM + i * 16 + 4 * h);
        const float sa[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc0[i][r] = sa[r] * sb0;
          sc1[i][r] = SWIGLU ? sa[r] * sb1 : 0.f;
        }
      }
    }
    v8i a[C_::SI];
#pragma unroll
    for (int i = 0; i < C_::SI; ++i) a[i] = lds_frag(tA, wm * C_::WTM + i * 16 + (lane & 15), h);
    if (EXACT && c_rows > 16) {
      // exact sums, for tiles of more than one 16-row block (a tile of at
      // most 16 rows streams its weights at full rate in the single-
      // instruction form below): phase p of every (row block, column
      // subtile) pair, the pairs' chains interleaved (independent
      // accumulators), the step's copies spread over the phases; then one
      // promotion FMA per output
      v8i bb[C_::SJ];
#pragma unroll
      for (int j = 0; j < C_::SJ; ++j) bb[j] = b_frag(tB, j);
      v4f pc[C_::SI][C_::SJ];
#pragma unroll
      for (int i = 0; i < C_::SI; ++i)
#pragma unroll
        for (int j = 0; j < C_::SJ; ++j) pc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
#pragma unroll
        for (int i = 0; i < C_::SI; ++i) {
          if (i > 0 && wm * C_::WTM + 16 * i >= c_rows) continue;
          const v8i x = exact_phase(a[i], p);
#pragma unroll
          for (int j = 0; j < C_::SJ; ++j) pc[i][j] = mfma_fp8(x, bb[j], pc[i][j]);
        }
        if (do_issue) {
#pragma unroll
          for (int k = (p * C_::LOADS) / 8; k < ((p + 1) * C_::LOADS) / 8; ++k) issue_op(k);
        }
      }
      if (do_issue) issue_end();
#pragma unroll
      for (int j = 0; j < C_::SJ; ++j) {
        const bool up = SWIGLU && j >= SJH;
#pragma unroll
        for (int i = 0; i < C_::SI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = fmaf(up ? sc1[i][r] : sc0[i][r], pc[i][j][r], acc[i][j][r]);
      }
    } else {
      // software pipeline over column subtiles: the MFMAs of subtile j and the
      // LDS read of j+1 are issued before the promotion FMAs of subtile j-1
      v8i bcur = b_frag(tB, 0);
      v4f pprev[C_::SI];
#pragma unroll
      for (int j = 0; j < C_::SJ; ++j) {
        v8i bnext = bcur;
        if (j + 1 < C_::SJ) bnext = b_frag(tB, j + 1);
        // row blocks wholly past the group's end are never stored: no MFMAs
        v4f pcur[C_::SI];
#pragma unroll
        for (int i = 0; i < C_::SI; ++i) {
          if (i == 0 || wm * C_::WTM + 16 * i < c_rows)
            pcur[i] = mfma_fp8_block(a[i], bcur);
          else
            pcur[i] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        if (do_issue) {
          // copies k in [j*LOADS/SJ, (j+1)*LOADS/SJ) of the step STAGES-1 ahead
#pragma unroll
          for (int k = (j * C_::LOADS) / C_::SJ; k < ((j + 1) * C_::LOADS) / C_::SJ; ++k) issue_op(k);
        }
        if (j > 0) {
          const bool up = SWIGLU && (j - 1) >= SJH;
#pragma unroll
          for (int i = 0; i < C_::SI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i][j - 1][r] = fmaf(up ? sc1[i][r] : sc0[i][r], pprev[i][r], acc[i][j - 1][r]);
        }
#pragma unroll
        for (int i = 0; i < C_::SI; ++i) pprev[i] = pcur[i];
        bcur = bnext;
      }
      if (do_issue) issue_end();
      {
        const bool up = SWIGLU && (C_::SJ - 1) >= SJH;
#pragma unroll
        for (int i = 0; i < C_::SI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][C_::SJ - 1][r] =
                fmaf(up ? sc1[i][r] : sc0[i][r], pprev[i][r], acc[i][C_::SJ - 1][r]);
      }
    }

    const int ct = c_ord;
    const bool tile_done = (c_kb == nkb32 - 1);
    if (++slot == STAGES) slot = 0;
    if (++c_kb == nkb32) {
      c_kb = 0;
      ++c_ord;
    }
    if (!tile_done) continue;

    // ---- epilogue of tile ct (from registers) ----
    const Tile t = tile_of(ct);
    if (!SWIGLU) {
      // bf16 (round to nearest even); the 4 lanes of a quad hold 4
      // consecutive columns of a row, lane 4k stores them as one 8-byte word
#pragma unroll
      for (int i = 0; i < C_::SI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = (int64_t)t.m0 + wm * C_::WTM + i * 16 + 4 * h + r;
          const bool ok = row < t.m1 && (lane & 3) == 0;
#pragma unroll
          for (int j = 0; j < C_::SJ; ++j) {
            const float v0 = acc[i][j][r];
            const float v1 = quad_lane1(v0), v2 = quad_lane2(v0), v3 = quad_lane3(v0);
            const int64_t col = 256 * t.nt + wn * C_::WTN + j * 16 + (lane & 15);
            if (ok && col < N)
              *reinterpret_cast<uint2*>(args.C + row * N + col) =
                  make_uint2(f32x2_to_bf16x2(v0, v1), f32x2_to_bf16x2(v2, v3));
          }
        }
    } else {
      // h = silu(g) * u per (row, h column): gate subtile j pairs with up
      // subtile j + SJ/2 in this lane's registers.  exp and the reciprocal
      // use the hardware v_exp_f32 / v_rcp_f32 (a few ulp; h feeds a 3-bit
      // mantissa code).
      float* s_amax = reinterpret_cast<float*>(smem + C_::OFF_AMAX);
#pragma unroll
      for (int i = 0; i < C_::SI; ++i)
#pragma unroll
        for (int j = 0; j < SJH; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = acc[i][j][r], u = acc[i][j + SJH][r];
            const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
            const float a = g * __builtin_amdgcn_rcpf(1.0f + e);
            acc[i][j][r] = a * u;
          }
#pragma unroll
      for (int i = 0; i < C_::SI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < SJH; ++j) m = fmaxf(m, fabsf(acc[i][j][r]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          if ((lane & 15) == 0) s_amax[(wm * C_::WTM + i * 16 + 4 * h + r) * C_::WAVES_N + wn] = m;
        }
      wait_lgkm0();
      barrier();
#pragma unroll
      for (int i = 0; i < C_::SI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int trow = wm * C_::WTM + i * 16 + 4 * h + r;
          float amax = 0.f;
#pragma unroll
          for (int w = 0; w < C_::WAVES_N; ++w) amax = fmaxf(amax, s_amax[trow * C_::WAVES_N + w]);
          const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
          const float inv = 1.0f / sc;
          const int64_t row = (int64_t)t.m0 + trow;
          const bool ok = row < t.m1;
#pragma unroll
          for (int j = 0; j < SJH; ++j) {
            const float v0 = acc[i][j][r] * inv;
            const float v1 = quad_lane1(v0), v2 = quad_lane2(v0), v3 = quad_lane3(v0);
            const int64_t col = 128 * t.nt + wn * WHN + 16 * j + (lane & 15);
            if (ok && (lane & 3) == 0)
              *reinterpret_cast<uint32_t*>(args.Hq + row * args.I + col) =
                  f32x4_to_e4m3x4(v0, v1, v2, v3);
          }
          if (ok && wn == 0 && (lane & 15) == 0) args.Hs[row * (args.I >> 7) + t.nt] = sc;
        }
    }
#pragma unroll
    for (int i = 0; i < C_::SI; ++i)
#pragma unroll
      for (int j = 0; j < C_::SJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

}  // namespace

int num_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

namespace {

template <int BM, int WAVES_M, int STAGES, bool SWIGLU, bool EXACT = false>
int launch(const GemmArgs& a, hipStream_t st) {
  const int grid = std::max(8, (num_cus() / 8) * 8);
  if (a.a_row_index)
    grouped_gemm_kernel<BM, WAVES_M, STAGES, SWIGLU, true, EXACT>
        <<<dim3(grid), dim3(GM_THREADS), 0, st>>>(a);
  else
    grouped_gemm_kernel<BM, WAVES_M, STAGES, SWIGLU, false, EXACT>
        <<<dim3(grid), dim3(GM_THREADS), 0, st>>>(a);
  return MOE_OK;
}

// the input-gradient form (B = W in its forward layout): same tile shapes
template <int BM, int WAVES_M, int STAGES>
int launch_bt(const GemmArgs& a, hipStream_t st) {
  const int grid = std::max(8, (num_cus() / 8) * 8);
  grouped_gemm_kernel<BM, WAVES_M, STAGES, false, false, false, true>
      <<<dim3(grid), dim3(GM_THREADS), 0, st>>>(a);
  return MOE_OK;
}

// the 256x256 kernel: groups of at least 160 rows on average; it addresses
// a tile's output, A and one group's B with 32-bit offsets, and takes an
// even number of at least 6 K blocks
template <bool SWIGLU>
bool takes_wide(const GemmArgs& a, int64_t M_total) {
  const int64_t avg = M_total / a.G;
  const int64_t nkb = a.K / 128;
  const int64_t lim = (int64_t)1 << 32;
  const bool wide_ok = (SWIGLU ? a.I <= (1 << 22) : (a.N % 256 == 0 && a.N <= (1 << 21))) &&
                       nkb >= 6 && nkb % 2 == 0 && a.K <= (1 << 20) && a.N * a.K < lim &&
                       a.A_rows * a.K < lim;
  return avg >= 160 && wide_ok;
}

template <bool SWIGLU>
int dispatch(const GemmArgs& a, int64_t M_total, hipStream_t st) {
  // rows per group decide the M tile: 256 (the wide kernel) or 128 for
  // prefill-sized groups, 32 when groups hold a handful of rows (decode), 64
  // in between.  The 32-row launches are bound by their weight stream (a few
  // rows per 128x128 weight block); in those feeding the SwiGLU
  // requantisation, tiles of more than 16 rows (at decode: the shared
  // expert, which every token adds with weight one) take the exact-sum MFMA
  // form, which removes the truncation error of their gate/up sums; tiles of
  // at most 16 rows and the plain bf16 launches keep the full-rate form.
  const int64_t avg = M_total / a.G;
  if (takes_wide<SWIGLU>(a, M_total)) return launch_wide(a, SWIGLU, st);
  if (avg >= 96) return launch<128, 2, 3, SWIGLU>(a, st);
  if (avg >= 40) return launch<64, 1, 3, SWIGLU>(a, st);
  return launch<32, 1, 4, SWIGLU, SWIGLU>(a, st);
}

int validate_common(const char* who, const uint8_t* A, const float* A_scale,
                    const int32_t* a_row_index, int64_t A_rows, const uint8_t* B,
                    const float* B_scale, const int32_t* group_offsets, int32_t G,
                    int64_t M_total, int64_t N, int64_t K) {
  MOE_INVALID(G >= 1, "%s: G=%d must be >= 1", who, (int)G);
  MOE_UNSUPPORTED(G <= MAXG, "%s: G=%d > %d groups is not supported", who, (int)G, MAXG);
  MOE_INVALID(M_total >= 0 && M_total < (1ll << 31), "%s: M_total=%lld out of range", who,
              (long long)M_total);
  MOE_INVALID(N > 0 && N % 128 == 0, "%s: N=%lld must be a positive multiple of 128", who,
              (long long)N);
  MOE_INVALID(K > 0 && K % 128 == 0, "%s: K=%lld must be a positive multiple of 128", who,
              (long long)K);
  if (M_total == 0) return MOE_OK;
  MOE_INVALID(A_rows >= (a_row_index ? 1 : M_total) && A_rows < (1ll << 31),
              "%s: A_rows=%lld must be in [%s, 2^31)", who, (long long)A_rows,
              a_row_index ? "1" : "M_total");
  MOE_INVALID(A && A_scale && B && B_scale && group_offsets, "%s: null pointer", who);
  MOE_INVALID(((uintptr_t)A & 15) == 0 && ((uintptr_t)B & 15) == 0 &&
                  ((uintptr_t)A_scale & 3) == 0 && ((uintptr_t)B_scale & 3) == 0,
              "%s: A and B must be 16-byte aligned, scales 4-byte aligned", who);
  return MOE_OK;
}

}  // namespace
}  // namespace gemm
}  // namespace moe

using namespace moe;
using namespace moe::gemm;

extern "C" int grouped_fp8_gemm(const uint8_t* A, const float* A_scale, const int32_t* a_row_index,
                                int64_t A_rows, const uint8_t* B, const float* B_scale,
                                const int32_t* group_offsets, int32_t G, int64_t M_total, int64_t N,
                                int64_t K, void* C_bf16, void* stream) {
  clear_error();
  int rc = validate_common("grouped_fp8_gemm", A, A_scale, a_row_index, A_rows, B, B_scale,
                           group_offsets, G, M_total, N, K);
  if (rc != MOE_OK || M_total == 0) return rc;
  MOE_INVALID(C_bf16 && ((uintptr_t)C_bf16 & 15) == 0,
              "grouped_fp8_gemm: C must be non-null and 16-byte aligned");
  GemmArgs a{};
  a.A = A; a.A_scale = A_scale; a.a_row_index = a_row_index; a.A_rows = A_rows;
  a.B = B; a.B_scale = B_scale;
  a.offs = group_offsets; a.G = G; a.N = N; a.K = K; a.ntiles = ceil_div(N, BN); a.I = 0;
  a.C = static_cast<uint16_t*>(C_bf16);
  rc = dispatch<false>(a, M_total, as_stream(stream));
  if (rc != MOE_OK) return rc;
  return check_launch("grouped_fp8_gemm");
}

extern "C" int grouped_fp8_gemm_dgrad(const uint8_t* dC, const float* dC_scale,
                                      const uint8_t* W, const float* W_scale,
                                      const int32_t* group_offsets, int32_t G, int64_t M_total,
                                      int64_t N, int64_t K, void* dA_bf16, void* stream) {
  clear_error();
  // the kernel contracts over N (W's rows) and writes K columns
  int rc = validate_common("grouped_fp8_gemm_dgrad", dC, dC_scale, nullptr, M_total, W, W_scale,
                           group_offsets, G, M_total, K, N);
  if (rc != MOE_OK || M_total == 0) return rc;
  MOE_INVALID(dA_bf16 && ((uintptr_t)dA_bf16 & 15) == 0,
              "grouped_fp8_gemm_dgrad: dA must be non-null and 16-byte aligned");
  GemmArgs a{};
  a.A = dC; a.A_scale = dC_scale; a.a_row_index = nullptr; a.A_rows = M_total;
  a.B = W; a.B_scale = W_scale;
  a.offs = group_offsets; a.G = G; a.N = K; a.K = N; a.ntiles = ceil_div(K, BN); a.I = 0;
  a.C = static_cast<uint16_t*>(dA_bf16);
  // tile shape by rows per group, as in grouped_fp8_gemm; the 256x256 kernel
  // also needs whole 256-column tiles and 32-bit copy offsets
  hipStream_t st = as_stream(stream);
  const int64_t avg = M_total / G, lim = (int64_t)1 << 32;
  const bool wide_ok = K % 256 == 0 && K <= (1 << 21) && N % 256 == 0 && N >= 768 &&
                       N <= (1 << 20) && N * K < lim && M_total * N < lim;
  if (avg >= 160 && wide_ok) rc = launch_wide_bt(a, st);
  else if (avg >= 96) rc = launch_bt<128, 2, 3>(a, st);
  else if (avg >= 40) rc = launch_bt<64, 1, 3>(a, st);
  else rc = launch_bt<32, 1, 4>(a, st);
  if (rc != MOE_OK) return rc;
  return check_launch("grouped_fp8_gemm_dgrad");
}

extern "C" int grouped_fp8_gemm_swiglu(const uint8_t* A, const float* A_scale,
                                       const int32_t* a_row_index, int64_t A_rows, const uint8_t* B,
                                       const float* B_scale, const int32_t* group_offsets,
                                       int32_t G, int64_t M_total, int64_t I, int64_t K,
                                       uint8_t* H_e4m3, float* H_scale, void* stream) {
  clear_error();
  MOE_INVALID(I > 0 && I % 128 == 0, "grouped_fp8_gemm_swiglu: I=%lld must be a positive "
              "multiple of 128", (long long)I);
  int rc = validate_common("grouped_fp8_gemm_swiglu", A, A_scale, a_row_index, A_rows, B,
                           B_scale, group_offsets, G, M_total, 2 * I, K);
  if (rc != MOE_OK || M_total == 0) return rc;
  MOE_INVALID(H_e4m3 && H_scale && ((uintptr_t)H_e4m3 & 15) == 0,
              "grouped_fp8_gemm_swiglu: H must be non-null and 16-byte aligned");
  GemmArgs a{};
  a.A = A; a.A_scale = A_scale; a.a_row_index = a_row_index; a.A_rows = A_rows;
  a.B = B; a.B_scale = B_scale;
  a.offs = group_offsets; a.G = G; a.N = 2 * I; a.K = K; a.ntiles = I / 128; a.I = I;
  a.Hq = H_e4m3; a.Hs = H_scale;
  rc = dispatch<true>(a, M_total, as_stream(stream));
  if (rc != MOE_OK) return rc;
  return check_launch("grouped_fp8_gemm_swiglu");
}

extern "C" int grouped_fp8_gemm_swiglu_keep(const uint8_t* A, const float* A_scale,
                                            const int32_t* a_row_index, int64_t A_rows,
                                            const uint8_t* B, const float* B_scale,
                                            const int32_t* group_offsets, int32_t G,
                                            int64_t M_total, int64_t I, int64_t K,
                                            uint8_t* H_e4m3, float* H_scale, void* GU_bf16,
                                            void* stream) {
  clear_error();
  MOE_INVALID(I > 0 && I % 128 == 0, "grouped_fp8_gemm_swiglu_keep: I=%lld must be a positive "
              "multiple of 128", (long long)I);
  int rc = validate_common("grouped_fp8_gemm_swiglu_keep", A, A_scale, a_row_index, A_rows, B,
                           B_scale, group_offsets, G, M_total, 2 * I, K);
  if (rc != MOE_OK || M_total == 0) return rc;
  MOE_INVALID(H_e4m3 && H_scale && ((uintptr_t)H_e4m3 & 15) == 0,
              "grouped_fp8_gemm_swiglu_keep: H must be non-null and 16-byte aligned");
  MOE_INVALID(GU_bf16 && ((uintptr_t)GU_bf16 & 15) == 0,
              "grouped_fp8_gemm_swiglu_keep: GU must be non-null and 16-byte aligned");
  GemmArgs a{};
  a.A = A; a.A_scale = A_scale; a.a_row_index = a_row_index; a.A_rows = A_rows;
  a.B = B; a.B_scale = B_scale;
  a.offs = group_offsets; a.G = G; a.N = 2 * I; a.K = K; a.ntiles = I / 128; a.I = I;
  a.Hq = H_e4m3; a.Hs = H_scale;
  hipStream_t st = as_stream(stream);
  if (takes_wide<true>(a, M_total)) {
    a.GU = static_cast<uint16_t*>(GU_bf16);  // the fused kernel writes both
    rc = launch_wide(a, true, st);
  } else {
    // smaller groups: the fused kernel, then the plain GEMM for the sums
    rc = dispatch<true>(a, M_total, st);
    if (rc == MOE_OK) {
      GemmArgs p{};
      p.A = A; p.A_scale = A_scale; p.a_row_index = a_row_index; p.A_rows = A_rows;
      p.B = B; p.B_scale = B_scale;
      p.offs = group_offsets; p.G = G; p.N = 2 * I; p.K = K; p.ntiles = ceil_div(2 * I, BN);
      p.C = static_cast<uint16_t*>(GU_bf16);
      rc = dispatch<false>(p, M_total, st);
    }
  }
  if (rc != MOE_OK) return rc;
  return check_launch("grouped_fp8_gemm_swiglu_keep");
}
