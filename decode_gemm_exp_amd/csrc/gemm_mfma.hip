// gemm_mfma.hip -- reconstructive bf16 MFMA GEMM for gfx950, y = x . W^T from
// BF16, exponent + sign/mantissa, or palette + sign/mantissa weights, stored
// W[N][K] (NK) or W^T[K][N] (KN).
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "重建矩陣乘法核心運作": the
// matmul streams compressed weight tiles from HBM into on-chip memory, rebuilds
// BF16 there and feeds the matrix units, so rebuilt weights never return to
// HBM.  Section "Llama 3.1 8B測試結果" names the cost this design has to hide:
// every weight tile is rebuilt once per tile of batch rows.
//
// Structure (4 or 8 waves in a WGM x WGN grid, tile BM x BN, K step 64):
//   * the x tile and the rebuilt weight tile live in LDS, double buffered,
//     one barrier per step;
//   * step s: the waves run the MFMAs of step s from one buffer while, in the
//     same instruction stream, every thread rebuilds step s+1 from registers
//     into the other buffer and requests the raw data of step s+2 (x rows and
//     compressed weights); for the palette format the verbatim flag words are
//     loaded one step earlier still, so the side-section address of a
//     verbatim group is known when its data is requested;
//   * each weight is rebuilt once per block (not once per wave) straight into
//     LDS with 16-byte stores: NK tiles n-major, KN tiles k-major; KN B
//     fragments come from the k-major tile through transposing LDS reads
//     (ds_read_b64_tr_b16), so no 16-bit scatter is needed;
//   * waves read A and B fragments from LDS and issue v_mfma_f32_32x32x16_bf16;
//   * block order is XCD-aware (see block_tile);
//   * split K: grid.z slices of K write partial tiles to the workspace and a
//     fixed-order reduction adds them (deterministic).
#include <cstring>

#include "rebuild.h"

namespace uw {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;   // bf16 per LDS row: 144 bytes keeps 16-byte alignment, spreads banks

// Raw compressed data of one 16-weight chunk, as loaded from HBM.
struct Raw {
  uint4 a;      // bf16: weights 0..7 | exp/pal: 16 sign+mantissa bytes
  uint4 b;      // bf16: weights 8..15 | exp: 16 exponent bytes | pal: the aligned 16 index
                //   bytes holding the chunk's 8, or its 16 verbatim exponent bytes
};

// Raw loads of one chunk.  Straight-line code: a chunk outside the matrix
// reads chunk 0 instead (valid memory) and is zeroed when rebuilt, so that the
// loads, the rebuild and the MFMAs of a step stay in one basic block for the
// scheduler to interleave.
template <int FMT>
__device__ __forceinline__ void load_raw(const WeightView& w, uint64_t el, bool valid, uint32_t flagword,
                                         uint32_t rankword, Raw& r) {
  el = valid ? el : 0;
  if constexpr (FMT == kFmtBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(w.bf16 + el);
    r.a = p[0];
    r.b = p[1];
  } else if constexpr (FMT == kFmtExp) {
    r.a = *reinterpret_cast<const uint4*>(w.sm + el);
    r.b = *reinterpret_cast<const uint4*>(w.ex + el);
  } else {
    r.a = *reinterpret_cast<const uint4*>(w.sm + el);
    const uint64_t g = el >> 6;
    const uint8_t* p = valid && group_verbatim(flagword, g)
                           ? w.vexp + (uint64_t)group_rank(flagword, rankword, g) * 64 + (el & 63)
                           : w.pidx + ((el >> 1) & ~(uint64_t)15);
    r.b = *reinterpret_cast<const uint4*>(p);
  }
}

// Rebuild 16 weights (8 dwords of packed bf16) from a raw chunk; chunks
// outside the matrix give exact zeros (a K tail multiplies them by zero x).
template <int FMT>
__device__ __forceinline__ void rebuild_raw(const WeightView& w, const Raw& r, bool valid, bool verbatim, bool hi,
                                            uint32_t o[8]) {
  if constexpr (FMT == kFmtBf16) {
    o[0] = r.a.x; o[1] = r.a.y; o[2] = r.a.z; o[3] = r.a.w;
    o[4] = r.b.x; o[5] = r.b.y; o[6] = r.b.z; o[7] = r.b.w;
  } else if constexpr (FMT == kFmtExp) {
    rebuild16(r.a, r.b, o);
  } else {
    uint4 e = pal16<FMT == kFmtPalRun>(hi ? r.b.z : r.b.x, hi ? r.b.w : r.b.y, w.pal);
    if (verbatim) e = r.b;
    rebuild16(r.a, e, o);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = valid ? o[i] : 0u;
}

typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// B fragment (32 columns x 16 k) from a k-major LDS tile [k][n] through two
// transposing reads: in each 16-lane group, source lane s addresses row
// k + s/4 and columns c + 4 (s % 4); lane i of the group then holds column
// c + i of those 4 rows.  Group g covers columns 16 (g & 1) and k rows
// 8 (g >> 1), which is the v_mfma_f32_32x32x16_bf16 B operand layout.
__device__ __forceinline__ bf16x8 b_frag_kmajor(const uint16_t* wt, int ldw, int kk, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = kk + 8 * (g >> 1) + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(wt + row * ldw + col));
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(wt + (row + 4) * ldw + col));
  typedef __attribute__((ext_vector_type(8))) short v8i16;
  const v8i16 v = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Tile of a block: when the N tiles split evenly over the 8 XCDs (blocks are
// dealt to XCDs round-robin), all M tiles of an N tile run on one XCD, one
// after another, so its L2 serves the rebuilt-weight tile's compressed data to
// every M tile and the 32 blocks resident on an XCD share x rows.
__device__ __forceinline__ void block_tile(int b, int ntiles, int mtiles, int& nt, int& mt) {
  if ((ntiles & 7) == 0) {
    const int xcd = b & 7, l = b >> 3;
    nt = xcd + 8 * (l / mtiles);
    mt = l % mtiles;
  } else {
    nt = b / mtiles;
    mt = b % mtiles;
  }
}

template <int LAYOUT, int BN>
constexpr int w_ld() { return LAYOUT == 0 ? kLDK : BN + 16; }   // KN rows: BN + 16 keeps transposing reads conflict-light
template <int LAYOUT, int BN>
constexpr int w_tile_elems() { return LAYOUT == 0 ? BN * kLDK : kBK * (BN + 16); }

// NW waves per block (4 or 8); with 8 two waves share each SIMD, so one
// wave's rebuild arithmetic can issue while the other's MFMAs run.
// One launch serves a group of up to four matrices with the same K, layout
// and format.  Grid x holds every matrix's tiles back to back (matrix g from
// block bstart[g]), so no block is idle and the hardware's round-robin deal
// of blocks to XCDs spreads each matrix evenly.  Matrix g writes columns
// ycol[g].. of y, or columns pcol[g].. of the partial rows (pld wide) when K
// is split.
template <int LAYOUT, int FMT, int BM, int BN, int WGM, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_mfma2(Mfma2Group grp, const uint16_t* __restrict__ x, int B,
                                                   float* __restrict__ y, int64_t ldy, int64_t kslice,
                                                   float* __restrict__ part, int64_t pld, int mtiles) {
  constexpr int NT = 64 * NW;
  constexpr int WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int XC = BM * 8 / NT;      // 16-byte x chunks per thread per step
  constexpr int WC = BN * 4 / NT;      // 16-weight chunks per thread per step
  constexpr int LDW = w_ld<LAYOUT, BN>();
  constexpr int XS = BM * kLDK, WS = w_tile_elems<LAYOUT, BN>();
  constexpr int kValuPerMfma = FMT == kFmtBf16 ? 1 : 4;
  static_assert(TM >= 1 && TN >= 1 && XC >= 1 && WC >= 1, "tile too small");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  int g = 0;
  while (g + 1 < grp.count && (int)blockIdx.x >= grp.bstart[g + 1]) ++g;
  const int ntiles = grp.ntiles[g];
  const WeightView w = grp.w[g];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t N = (int64_t)w.n, K = (int64_t)w.k;
  int nt, mt;
  block_tile((int)blockIdx.x - grp.bstart[g], ntiles, mtiles, nt, mt);
  const int64_t n0 = (int64_t)nt * BN, m0 = (int64_t)mt * BM;
  const int64_t kb = (int64_t)blockIdx.z * kslice;
  const int64_t ke = kb + kslice < K ? kb + kslice : K;
  const int steps = (int)((ke - kb + kBK - 1) / kBK);

  // chunk c of this thread (i-th): NK -> row r = c / 4, k sub-block q = c % 4;
  // KN -> k row kr = c / (BN/16), n sub-block q = c % (BN/16)
  auto chunk_el = [&](int i, int64_t k0, bool& valid) __attribute__((always_inline)) -> uint64_t {
    const int c = tid + i * NT;
    if constexpr (LAYOUT == 0) {
      const int64_t n = n0 + (c >> 2), k = k0 + (c & 3) * 16;
      valid = n < N && k < ke;
      return (uint64_t)(n * K + k);
    } else {
      constexpr int QN = BN / 16;
      const int64_t k = k0 + c / QN, n = n0 + (c % QN) * 16;
      valid = k < ke && n < N;
      return (uint64_t)(k * N + n);
    }
  };

  uint4 xr[XC];
  Raw wr[WC];
  bool wverb[WC], wval[WC], whi[WC];
  uint32_t fw_a[WC], rk_a[WC];   // palette: flag / rank words of the step whose data loads next

  // The per-step work is split into four parts (one per 16-wide k slice of
  // the MFMAs); chunk i of the loads and stores belongs to part (4 i) / n.
  auto in_part = [](int i, int n, int part) __attribute__((always_inline)) { return (4 * i) / n == part; };
  auto load_flags = [&](int64_t k0, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      if (!in_part(i, WC, part)) continue;
      bool v;
      const uint64_t el = chunk_el(i, k0, v);
      const uint64_t fi = v ? el >> 11 : 0;
      const uint32_t f = w.vflags[fi], r = w.vrank[fi];
      fw_a[i] = v ? f : 0u;
      rk_a[i] = v ? r : 0u;
    }
  };
  auto load_step = [&](int64_t k0, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      if (!in_part(i, XC, part)) continue;
      // rows past the batch are never stored and k past the slice meets zeroed
      // weight rows, so x needs only a clamped (always valid) address
      const int c = tid + i * NT;
      const int64_t row0 = m0 + (c >> 3), kk0 = k0 + (c & 7) * 8;
      const int64_t row = row0 < B ? row0 : B - 1, kk = kk0 < K ? kk0 : K - 8;
      const uint4 t = *reinterpret_cast<const uint4*>(x + row * K + kk);
      xr[i] = t;
    }
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      if (!in_part(i, WC, part)) continue;
      bool v;
      const uint64_t el = chunk_el(i, k0, v);
      load_raw<FMT>(w, el, v, fw_a[i], rk_a[i], wr[i]);
      // zeroed when rebuilt: only [K][N] chunks past K.  Chunks past N only
      // feed output columns that are never stored, and a stored [N][K] row is
      // a multiple of 64 long, so none of its steps that are read reach past K
      if constexpr (LAYOUT == 0) {
        wval[i] = true;
      } else {
        wval[i] = k0 + (int64_t)((tid + i * NT) / (BN / 16)) < ke;
      }
      wverb[i] = fmt_is_pal(FMT) && v && group_verbatim(fw_a[i], el >> 6);
      whi[i] = (el & 16) != 0;
    }
  };
  // registers of a step -> LDS buffer (x as is, weights rebuilt)
  auto store_step = [&](uint16_t* xs, uint16_t* ws, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      if (!in_part(i, XC, part)) continue;
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&xs[(c >> 3) * kLDK + (c & 7) * 8]) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      if (!in_part(i, WC, part)) continue;
      uint32_t o[8];
      rebuild_raw<FMT>(w, wr[i], wval[i], wverb[i], whi[i], o);
      const int c = tid + i * NT;
      uint4* d;
      if constexpr (LAYOUT == 0) {
        d = reinterpret_cast<uint4*>(&ws[(c >> 2) * kLDK + (c & 3) * 16]);
      } else {
        constexpr int QN = BN / 16;
        d = reinterpret_cast<uint4*>(&ws[(c / QN) * LDW + (c % QN) * 16]);
      }
      d[0] = make_uint4(o[0], o[1], o[2], o[3]);
      d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragments of one 16-wide k slice, two sets: the next slice is read from
  // LDS while the MFMAs of the current one issue
  bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  auto read_frags = [&](const uint16_t* xs, const uint16_t* ws, int kk, bf16x8 (&a)[TM],
                        bf16x8 (&b)[TN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + i * 32 + (lane & 31);
      a[i] = *reinterpret_cast<const bf16x8*>(&xs[row * kLDK + kk + 8 * (lane >> 5)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (LAYOUT == 0) {
        const int col = wn * WN + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8*>(&ws[col * kLDK + kk + 8 * (lane >> 5)]);
      } else {
        b[j] = b_frag_kmajor(ws, LDW, kk, wn * WN + j * 32, lane);
      }
    }
  };
  auto mfma_set = [&](const bf16x8 (&a)[TM], const bf16x8 (&b)[TN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };

  uint16_t* const xs0 = lds;
  uint16_t* const xs1 = lds + XS;
  uint16_t* const ws0 = lds + 2 * XS;
  uint16_t* const ws1 = lds + 2 * XS + WS;

  // prologue: step 0 in LDS buffer 0, step 1 in registers, flags of step 2 loaded
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if constexpr (fmt_is_pal(FMT)) load_flags(kb, p);
    load_step(kb, p);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if constexpr (fmt_is_pal(FMT)) load_flags(kb + kBK, p);
    store_step(xs0, ws0, p);
    load_step(kb + kBK, p);
    if constexpr (fmt_is_pal(FMT)) load_flags(kb + 2 * kBK, p);
  }

  // step s: MFMAs from buffer s & 1 while step s+1 is rebuilt into the other
  // buffer and the raw data of step s+2 is requested; one barrier per step.
  // The last steps rebuild and load past the K range (clamped, zeroed, never
  // read) instead of branching, so every part is one basic block.
  auto body = [&](int st, const uint16_t* xs_c, const uint16_t* ws_c, uint16_t* xs_n, uint16_t* ws_n) __attribute__((always_inline)) {
    __syncthreads();
    const int64_t k2 = kb + (int64_t)(st + 2) * kBK, k3 = k2 + kBK;
    // part p: the MFMAs of k slice p (fragments read one part earlier), the
    // next slice's fragment reads, and a quarter of the next step's rebuild
    // and of the raw loads two steps ahead
    auto rest = [&](int p) __attribute__((always_inline)) {
      store_step(xs_n, ws_n, p);
      load_step(k2, p);
      if constexpr (fmt_is_pal(FMT)) load_flags(k3, p);
      // ask the scheduler to alternate one MFMA with a few VALU operations of
      // the rebuild, so the vector ALU works while the matrix core runs
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    read_frags(xs_c, ws_c, 0, fa0, fb0);
    read_frags(xs_c, ws_c, 16, fa1, fb1);
    mfma_set(fa0, fb0);
    rest(0);
    read_frags(xs_c, ws_c, 32, fa0, fb0);
    mfma_set(fa1, fb1);
    rest(1);
    read_frags(xs_c, ws_c, 48, fa1, fb1);
    mfma_set(fa0, fb0);
    rest(2);
    mfma_set(fa1, fb1);
    rest(3);
  };
  for (int st = 0; st < steps; ++st) {
    const bool odd = st & 1;
    body(st, odd ? xs1 : xs0, odd ? ws1 : ws0, odd ? xs0 : xs1, odd ? ws0 : ws1);
  }

  // ---- epilogue: y, or this K slice's partial tile part[slice][row][col] ----
  float* out = part ? part + (uint64_t)blockIdx.z * (uint64_t)B * (uint64_t)pld + grp.pcol[g] : y + grp.ycol[g];
  const int64_t ld = part ? pld : ldy;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
        if (row < B && col < N) out[row * ld + col] = acc[i][j][r];
      }
}

typedef void (*Mfma2Fn)(Mfma2Group, const uint16_t*, int, float*, int64_t, int64_t, float*, int64_t, int);

template <int L, int F>
Mfma2Fn pick(int tile) {
  switch (tile) {
    case 0: return k_mfma2<L, F, 64, 128, 2>;
    case 1: return k_mfma2<L, F, 128, 128, 2>;
    case 2: return k_mfma2<L, F, 128, 256, 2>;
    case 3: return k_mfma2<L, F, 256, 128, 2>;
    case 4: return k_mfma2<L, F, 256, 256, 2>;
    case 5: return k_mfma2<L, F, 32, 128, 1>;
    case 6: return k_mfma2<L, F, 32, 256, 1>;
    default: return k_mfma2<L, F, 256, 256, 2, 8>;
  }
}

}  // namespace

// Tiles of the big-tile kernel: {BM, BN}.
struct Tile2 {
  int bm, bn, waves;
};
// 32-row tiles (one MFMA row tile, four waves side by side) are for small
// batches; the last is 256x256 with eight waves (two per SIMD)
static const Tile2 kTiles2[] = {{64, 128, 4},  {128, 128, 4}, {128, 256, 4}, {256, 128, 4},
                                {256, 256, 4}, {32, 128, 4},  {32, 256, 4},  {256, 256, 8}};
int mfma2_tile_count() { return (int)(sizeof(kTiles2) / sizeof(kTiles2[0])); }
void mfma2_tile_dims(int tile, int* bm, int* bn) {
  *bm = kTiles2[tile].bm;
  *bn = kTiles2[tile].bn;
}

// K slices (powers of two, each slice >= 8 steps): until the grid covers the
// chip once, twice for the palette formats up to 64 rows, whose data loads
// wait on flag words and need a second resident block per CU to hide that.
// Tiles of 256 rows beyond 64 rows stop at the first split that fills seven
// eighths of the CUs instead: every slice adds a pass of B x N partial sums
// (70B gate at 256 rows, 112 tiles: 2 slices, 224 blocks, palette-direct
// 177 us against 203 us for the 4 slices that fill the chip; at 512 rows,
// 224 tiles: no split, 319 against 355 us).  Smaller tiles keep the full
// cover (palette-direct at 128 rows with 128x128 tiles: 149 us with 2
// slices, 187 us with none).
// LDS of one block: x and weight tiles, double buffered
size_t mfma2_lds_bytes(int layout, const Tile2& t) {
  const size_t wtile = layout == 0 ? (size_t)t.bn * kLDK : (size_t)kBK * (size_t)(t.bn + 16);
  return 2 * ((size_t)t.bm * kLDK + wtile) * sizeof(uint16_t);
}

int mfma2_slices(const WeightView& w, int64_t batch, int tile, int split_hint) {
  const Tile2 t = kTiles2[tile];
  const int64_t blocks = ((int64_t)w.n + t.bn - 1) / t.bn * ((batch + t.bm - 1) / t.bm);
  const int64_t cus = (int64_t)device_cus();
  const int64_t target = batch <= 64 ? (fmt_is_pal(w.fmt) ? 512 : 256) : t.bm >= 256 ? (cus * 7 + 7) / 8 : 256;
  // up to 64 rows, and for 256-row tiles up to 512 rows, never past the
  // blocks the CUs hold at once (a second round of blocks runs on a mostly
  // idle chip: 8B gate, palette-direct, 64 rows, 64x128 tiles: 4 slices
  // 40.6 us, 8 slices 47.7 us; 70B q+k+v grouped, 40 256x256 tiles at 192
  // rows: 4 slices 90 us, 8 slices 107 us; 8B q+k+v, 48 tiles at 384 rows:
  // 4 slices 52 us, 8 slices 66 us)
  const int64_t per_cu = (int64_t)(160 * 1024 / mfma2_lds_bytes((int)w.layout, t));
  const bool one_round = batch <= 64 || (t.bm >= 256 && batch <= 512);
  const int64_t hold = one_round ? cus * (per_cu > 0 ? per_cu : 1) : INT64_MAX;
  int s = split_hint > 0 ? split_hint : 1;
  if (split_hint <= 0)
    while (blocks * s < target && blocks * s * 2 <= hold && (int64_t)w.k / (64 * (s * 2)) >= 8) s *= 2;
  // beyond 64 rows, an unsplit palette grid that spills at most a quarter
  // round past whole rounds of resident blocks runs its last round of
  // full-length tiles on a mostly idle chip; two slices halve that tail
  // (70B q+k+v grouped, 640 128x128 tiles on 512 slots: 1024 rows 361 ->
  // 326 us, 896 rows 342 -> 319 us; 8B gate, 640 rows: 182 -> 173 us).
  // BF16 tiles run closer to the MFMA rate and lose more to the reduction
  // pass than the tail costs (the same three cases 5-10 % slower split).
  if (split_hint <= 0 && batch > 64 && s == 1 && fmt_is_pal(w.fmt)) {
    const int64_t slots = cus * (per_cu > 0 ? per_cu : 1), tail = blocks % slots;
    if (blocks > slots && tail > 0 && tail <= slots / 4 && (int64_t)w.k / (64 * 2) >= 8) s = 2;
  }
  const int64_t steps = ((int64_t)w.k + 63) / 64;
  if (s > steps) s = (int)steps;
  return s;
}

size_t mfma2_partial_elems(const WeightView& w, int64_t batch, int tile, int split_hint) {
  const int s = mfma2_slices(w, batch, tile, split_hint);
  return s > 1 ? (size_t)s * (size_t)batch * (size_t)w.n : 0;
}

// One launch over the group's tiles; K split as for one matrix as wide as the
// group, the partial rows group-wide so one reduction serves every matrix.
// The matrices' output columns in y must be consecutive from ycol[0].
static hipError_t launch_group(Mfma2Group grp, const uint16_t* x, int64_t batch, float* y, int64_t ldy,
                               int tile, int split_hint, float* part, size_t part_elems, hipStream_t s) {
  const Tile2 t = kTiles2[tile];
  const WeightView& w0 = grp.w[0];
  WeightView wide = w0;   // the group as one matrix: tiles, slices, partial rows
  int fmt = w0.fmt;
  uint64_t ntot = 0;
  const int mtiles = (int)((batch + t.bm - 1) / t.bm);
  int64_t nblocks = 0;
  for (int i = 0; i < grp.count; ++i) {
    ntot += grp.w[i].n;
    grp.bstart[i] = (int)nblocks;
    nblocks += (int64_t)grp.ntiles[i] * mtiles;
    if (grp.w[i].fmt != fmt) fmt = kFmtPal;   // palette kinds mixed: the general lookup
  }
  if (nblocks <= 0 || nblocks > INT32_MAX) return hipErrorInvalidValue;
  wide.n = ntot;
  wide.fmt = fmt;
  const int slices = mfma2_slices(wide, batch, tile, split_hint);
  const int64_t steps = ((int64_t)w0.k + 63) / 64;
  const int64_t kslice = ((steps + slices - 1) / slices) * 64;
  const bool split = slices > 1;
  if (split && (part == nullptr || part_elems < (size_t)slices * (size_t)batch * (size_t)ntot))
    return hipErrorInvalidValue;
  Mfma2Fn f;
  if (w0.layout == 0) {
    f = fmt == kFmtBf16 ? pick<0, kFmtBf16>(tile) : fmt == kFmtExp ? pick<0, kFmtExp>(tile)
        : fmt == kFmtPal ? pick<0, kFmtPal>(tile) : pick<0, kFmtPalRun>(tile);
  } else {
    f = fmt == kFmtBf16 ? pick<1, kFmtBf16>(tile) : fmt == kFmtExp ? pick<1, kFmtExp>(tile)
        : fmt == kFmtPal ? pick<1, kFmtPal>(tile) : pick<1, kFmtPalRun>(tile);
  }
  const size_t lds = mfma2_lds_bytes((int)w0.layout, t);
  {
    hipError_t e = allow_dynamic_lds((const void*)f, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)nblocks, 1, (unsigned)slices);
  hipLaunchKernelGGL(f, grid, dim3(64 * t.waves), lds, s, grp, x, (int)batch, y, ldy, kslice, split ? part : nullptr,
                     (int64_t)ntot, mtiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  return launch_sum_slices(part, slices, ntot, batch, y, ldy, grp.ycol[0], s);
}

hipError_t launch_mfma2(const WeightView& w, const uint16_t* x, int64_t batch, float* y, int64_t ldy, int64_t col0,
                        int tile, int split_hint, float* part, size_t part_elems, hipStream_t s) {
  Mfma2Group grp;
  std::memset(&grp, 0, sizeof(grp));
  grp.w[0] = w;
  grp.ycol[0] = col0;
  grp.pcol[0] = 0;
  grp.ntiles[0] = (int)((w.n + (uint64_t)kTiles2[tile].bn - 1) / (uint64_t)kTiles2[tile].bn);
  grp.count = 1;
  return launch_group(grp, x, batch, y, ldy, tile, split_hint, part, part_elems, s);
}

// 2..4 matrices of one layout, K and format class (palette kinds may mix),
// their outputs consecutive in y from col0s[0]
hipError_t launch_mfma2_group(const WeightView* ws, int count, const uint16_t* x, int64_t batch, float* y,
                              int64_t ldy, const int64_t* col0s, int tile, int split_hint, float* part,
                              size_t part_elems, hipStream_t s) {
  if (count < 2 || count > kMfma2GroupMax) return hipErrorInvalidValue;
  Mfma2Group grp;
  std::memset(&grp, 0, sizeof(grp));
  for (int i = 0; i < count; ++i) {
    if (ws[i].layout != ws[0].layout || ws[i].k != ws[0].k) return hipErrorInvalidValue;
    if (fmt_is_pal(ws[i].fmt) != fmt_is_pal(ws[0].fmt) || (!fmt_is_pal(ws[0].fmt) && ws[i].fmt != ws[0].fmt))
      return hipErrorInvalidValue;
    if (col0s[i] != col0s[0] + (i ? grp.pcol[i - 1] + (int64_t)ws[i - 1].n : 0)) return hipErrorInvalidValue;
    grp.w[i] = ws[i];
    grp.ycol[i] = col0s[i];
    grp.pcol[i] = col0s[i] - col0s[0];
    grp.ntiles[i] = (int)((ws[i].n + (uint64_t)kTiles2[tile].bn - 1) / (uint64_t)kTiles2[tile].bn);
  }
  grp.count = count;
  return launch_group(grp, x, batch, y, ldy, tile, split_hint, part, part_elems, s);
}

// partial floats of a group launch (0 when K is not split)
size_t mfma2_group_partial_elems(const WeightView* ws, int count, int64_t batch, int tile, int split_hint) {
  WeightView wide = ws[0];
  uint64_t ntot = 0;
  for (int i = 0; i < count; ++i) ntot += ws[i].n;
  wide.n = ntot;
  return mfma2_partial_elems(wide, batch, tile, split_hint);
}

}  // namespace uw
