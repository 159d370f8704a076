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

// Raw compressed data of one 16-weight chunk, as loaded from HBM.
struct Raw {
  uint4 a;      // bf16: weights 0..7 | exp/pal: 16 sign+mantissa bytes
  uint4 b;      // bf16: weights 8..15 | exp: 16 exponent bytes | pal: the aligned 16 index
                //   bytes holding the chunk's 8
  uint4 v;      // pal: the chunk's 16 verbatim exponent bytes (zero unless verbatim)
};

// Byte-addressed buffer resources: a read at or past the resource's end
// returns zero, so loads need neither clamps nor branches, and every load of
// a step sits in one basic block with the step's MFMAs.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
constexpr uint32_t kRecMax = 0x40000000u;     // a resource spans at most 1 GiB
constexpr uint32_t kPastEnd = 0x7FFF0000u;    // an offset past every resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)(bytes < kRecMax ? bytes : kRecMax), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t byte) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Weight data of a stored [K][N] tile: every step reads whole 128-byte lines
// of its rows, so the loads carry the non-temporal policy (32x256 tiles at 4
// to 32 rows of the 70B down projection: 7-8 % faster).  A stored [N][K]
// tile reads 64 bytes of each row per step and the rest of the line one step
// later, so its loads keep the line in the cache (non-temporal there: 10-28 %
// slower).
template <bool NT>
__device__ __forceinline__ uint4 bload16w(__amdgpu_buffer_rsrc_t r, uint32_t byte) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte, 0, NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t byte) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte, 0, 0);
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
    // a verbatim group's own exponents, selected without a branch so the
    // step stays one basic block
    const uint32_t vm = verbatim ? ~0u : 0u;
    e = make_uint4(bfi(vm, r.v.x, e.x), bfi(vm, r.v.y, e.y), bfi(vm, r.v.z, e.z), bfi(vm, r.v.w, e.w));
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

// bf16 per LDS row of an x tile or an [N][K] weight tile for a K step of
// 64 KW: 144 or 272 bytes keeps 16-byte alignment and spreads banks
constexpr int ld_k(int kw) { return kBK * kw + 8; }
template <int LAYOUT, int BN, int KW>
constexpr int w_ld() { return LAYOUT == 0 ? ld_k(KW) : BN + 16; }   // KN rows: BN + 16 keeps transposing reads conflict-light
template <int LAYOUT, int BN, int KW>
constexpr int w_tile_elems() { return LAYOUT == 0 ? BN * ld_k(KW) : kBK * (BN + 16); }

// x [B][K] -> the A fragments of v_mfma_f32_32x32x16_bf16 in the lanes'
// read order, for the tiles that keep x in registers: fragment (R, S) (rows
// 32 R.., columns 16 S..) is 1 KB at (R SK + S) KB with SK = ceil(K / 16), and
// lane l's 16 bytes are row 32 R + (l % 32), columns 16 S + 8 (l / 32) .. + 7.
// Each fragment load then reads 1 KB of contiguous memory instead of 32 rows
// of 32 bytes.  Rows past B and columns past K are zero.
__global__ __launch_bounds__(256) void k_pack_xa(const uint16_t* __restrict__ x, int B, int64_t K, int64_t SK,
                                                 int64_t pieces, uint4* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= pieces) return;
  const int64_t f = t >> 6;
  const int l = (int)(t & 63);
  const int64_t R = f / SK, S = f - R * SK;
  const int64_t row = 32 * R + (l & 31), col = 16 * S + 8 * (l >> 5);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < B && col < K) v = *reinterpret_cast<const uint4*>(x + row * K + col);   // K % 8 == 0
  out[t] = v;
}

// NW waves per block (4 or 8); with 8 two waves share each SIMD, so one
// wave's rebuild arithmetic can issue while the other's MFMAs run.
// One launch serves a group of up to four matrices with the same K, layout
// and format.  Grid x holds every matrix's tiles back to back (matrix g from
// block bstart[g]), so no block is idle and the hardware's round-robin deal
// of blocks to XCDs spreads each matrix evenly.  Matrix g writes columns
// ycol[g].. of y, or columns pcol[g].. of the partial rows (pld wide) when K
// is split.
//
// XREG (single rebuild): x never enters LDS.  Each wave owns BM / NW batch
// rows across the whole tile width and loads its MFMA A fragments straight
// from memory into registers, one k slice at a time, a step ahead; only the
// rebuilt weight tile is shared through LDS.  With BM = 512 every weight is
// rebuilt once per 512 batch rows (the 256-row tiles rebuild it once per 256),
// LDS carries a third less per MFMA, and the LDS tile is small.
template <int LAYOUT, int FMT, int BM, int BN, int WGM, int NW = 4, bool XREG = false, int KW = 1>
__global__ __launch_bounds__(64 * NW) void k_mfma2(Mfma2Group grp, const uint16_t* __restrict__ x, int B,
                                                   float* __restrict__ y, int64_t ldy, int64_t kslice,
                                                   float* __restrict__ part, int64_t pld, int mtiles) {
  constexpr int NT = 64 * NW;
  constexpr int WGN = NW / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int BK = kBK * KW;                   // k per step
  constexpr int LDK = ld_k(KW);
  constexpr int XPR = BK / 8, WPR = BK / 16;     // x chunks per x row, weight chunks per [N][K] row
  constexpr int XC = XREG ? 0 : BM * XPR / NT;   // 16-byte x chunks per thread per step (LDS-staged x)
  constexpr int WC = BN * 4 * KW / NT;           // 16-weight chunks per thread per step
  constexpr int LDW = w_ld<LAYOUT, BN, KW>();
  constexpr int XS = XREG ? 0 : BM * LDK, WS = w_tile_elems<LAYOUT, BN, KW>();
  static_assert(KW == 1 || LAYOUT == 0, "wide K steps: [N][K] tiles only");
  constexpr int kValuPerMfma = FMT == kFmtBf16 ? 1 : 4;
  static_assert(TM >= 1 && TN >= 1 && (XREG || XC >= 1) && WC >= 1, "tile too small");
  static_assert(!XREG || WGN == 1, "x in registers: a wave owns its rows across the tile width");
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
  const int steps = (int)((ke - kb + BK - 1) / BK);

  // Resources over what the block reads; offsets are 32-bit and advance by a
  // constant per step.  [N][K]: rows [n0, min(n0 + BN, N)) from column kb
  // (reads past the slice's K end belong to steps whose data is never
  // multiplied); [K][N]: rows [kb, ke) from column n0 (rows past ke read
  // zero, and are zeroed when rebuilt, since a K tail multiplies them).  The
  // host keeps every span under kRecMax.
  const uint64_t wbase = LAYOUT == 0 ? (uint64_t)n0 * (uint64_t)K + (uint64_t)kb
                                     : (uint64_t)kb * (uint64_t)N + (uint64_t)n0;
  const uint64_t wlim = LAYOUT == 0 ? (uint64_t)(n0 + BN < N ? n0 + BN : N) * (uint64_t)K
                                    : (uint64_t)ke * (uint64_t)N;
  const uint64_t wspan = wlim > wbase ? wlim - wbase : 0;
  const uint32_t wb32 = (uint32_t)wbase;   // element indices fit 32 bits (numel < 2^32)
  __amdgpu_buffer_rsrc_t rwa, rwb, rvx, rfl, rrk;
  if constexpr (FMT == kFmtBf16) {
    rwa = rsrc(w.bf16 + wbase, 2 * wspan);
    rwb = rwa;
  } else if constexpr (FMT == kFmtExp) {
    rwa = rsrc(w.sm + wbase, wspan);
    rwb = rsrc(w.ex + wbase, wspan);
  } else {
    rwa = rsrc(w.sm + wbase, wspan);
    rwb = rsrc(w.pidx + wbase / 2, (wspan + 1) / 2);
    rvx = rsrc(w.vexp, w.vexp_bytes);
    const uint64_t fwords = (w.n * w.k / 64 + 31) / 32;
    rfl = rsrc(w.vflags, 4 * fwords);
    rrk = rsrc(w.vrank, 4 * fwords);
  }
  // x as given ([B][K]), or XREG: packed into fragments (k_pack_xa) for the
  // mtiles x BM rows of the grid
  const int64_t SK = (K + 15) / 16;
  const __amdgpu_buffer_rsrc_t rx =
      XREG ? rsrc(x, (uint64_t)mtiles * (BM / 32) * (uint64_t)SK * 1024u) : rsrc(x, (uint64_t)B * (uint64_t)K * 2);
  constexpr int QN = BN / 16;
  // per step: a stored [N][K] chunk moves BK columns on, a [K][N] chunk 64 rows
  const uint32_t wadv = LAYOUT == 0 ? (uint32_t)BK : (uint32_t)kBK * (uint32_t)N;

  // chunk i of this thread (c = tid + i NT): [N][K] -> row c / WPR, columns
  // 16 (c % WPR) of the step; [K][N] -> k row c / QN, columns 16 (c % QN).
  // The chunks of one thread differ only in their row, by NT / WPR (or
  // NT / QN) rows, so one offset register serves all of them: wo = element offset of
  // chunk 0 in the step whose data loads next, chunk i at wo + i wstride.
  // The column within the row is the same for every chunk and every step
  // (steps move by multiples of 64 elements): whi = the chunk's 8 index bytes
  // are the upper half of their aligned 16, wsub = its offset in its group.
  static_assert(NT % WPR == 0 && NT % XPR == 0 && NT % QN == 0, "chunk columns must repeat across a thread's chunks");
  const uint32_t wstride = LAYOUT == 0 ? (uint32_t)(NT / WPR) * (uint32_t)K : (uint32_t)(NT / QN) * (uint32_t)N;
  uint32_t wo;
  int wkr;
  if constexpr (LAYOUT == 0) {
    wo = ((uint32_t)tid / WPR) * (uint32_t)K + 16u * ((uint32_t)tid % WPR);
    wkr = 16 * (int)((uint32_t)tid % WPR);   // the chunks' column in the step
  } else {
    wo = (uint32_t)(tid / QN) * (uint32_t)N + 16u * (uint32_t)(tid % QN);
    wkr = tid / QN;
  }
  const uint32_t wsub = (wb32 + wo) & 48u;
  const bool whi = (wsub & 16u) != 0;
  // x chunk i: row m0 + c / XPR, columns 8 (c % XPR) of the step, at xo + i
  // xstride bytes; rows past the batch read zero (never stored), columns past
  // K read the next row's values (finite; a K tail meets zeroed weight rows)
  const uint32_t xstride = (uint32_t)(NT / XPR) * (uint32_t)K * 2u;
  uint32_t xo = (uint32_t)((uint64_t)(m0 + (unsigned)tid / XPR) * (uint64_t)K + (uint64_t)kb + 8u * ((uint32_t)tid % XPR)) * 2u;
  int kstep = 0;   // k of the step whose data loads next, from kb
  const int klen = (int)(ke - kb);
  // XREG: this lane's piece of the packed A fragment (row fragment 0) of the
  // next four k slices to load; row fragment i is SK fragments on, slice s
  // one fragment (1 KB).  The registers hold four slices, a ring: slice s
  // runs from xa[s % 4], which then loads slice s + 4.
  uint32_t xao = 0;
  if constexpr (XREG)
    xao = (uint32_t)((((uint64_t)(m0 + wm * WM) / 32) * (uint64_t)SK + (uint64_t)kb / 16) * 1024u) +
          16u * (uint32_t)lane;
  const uint32_t xa_frag = (uint32_t)SK * 1024u;
  bf16x8 xa[4][TM];
  auto load_xa = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      xa[sl][i] = __builtin_bit_cast(bf16x8, bload16(rx, xao + (uint32_t)i * xa_frag + 1024u * (uint32_t)sl));
  };

  uint4 xr[XC > 0 ? XC : 1];
  Raw wr[WC];
  bool wverb[WC], wval[WC];
  uint32_t fw_a[WC], rk_a[WC];   // palette: flag / rank words of the step whose data loads next

  // The per-step work is split into four parts (one per 16-wide k slice of
  // the MFMAs); chunk i of the loads and stores belongs to part (4 i) / n.
  auto in_part = [](int i, int n, int part) __attribute__((always_inline)) { return (4 * i) / n == part; };
  // Flag and rank words of the step whose data loads next for the chunks of
  // `part`.  Called just after load_step(part) (after = true) that is the
  // step after the one wo points to, until part 3's load moves wo on.
  auto load_flags = [&](int part, bool after) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      if (!in_part(i, WC, part)) continue;
      const uint32_t next = after && part != 3 ? wadv : 0u;
      const uint32_t fo = ((wb32 + wo + next + (uint32_t)i * wstride) >> 11) * 4u;
      fw_a[i] = bload4(rfl, fo);
      rk_a[i] = bload4(rrk, fo);
    }
  };
  auto load_step = [&](int part) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      if (!in_part(i, XC, part)) continue;
      xr[i] = bload16(rx, xo + (uint32_t)i * xstride);
    }
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      if (!in_part(i, WC, part)) continue;
      const uint32_t o = wo + (uint32_t)i * wstride;
      if constexpr (FMT == kFmtBf16) {
        wr[i].a = bload16w<LAYOUT == 1>(rwa, 2u * o);
        wr[i].b = bload16w<LAYOUT == 1>(rwa, 2u * o + 16u);
      } else if constexpr (FMT == kFmtExp) {
        wr[i].a = bload16w<LAYOUT == 1>(rwa, o);
        wr[i].b = bload16w<LAYOUT == 1>(rwb, o);
      } else {
        const uint32_t bit = ((wb32 + o) >> 6) & 31u;
        const bool verb = (fw_a[i] >> bit) & 1u;
        const uint32_t rank = rk_a[i] + (uint32_t)__popc(fw_a[i] & ((1u << bit) - 1u));
        wr[i].a = bload16w<LAYOUT == 1>(rwa, o);
        wr[i].b = bload16w<LAYOUT == 1>(rwb, (o >> 1) & ~15u);
        wr[i].v = bload16w<LAYOUT == 1>(rvx, verb ? rank * 64u + wsub : kPastEnd);
        wverb[i] = verb;
      }
      // zeroed when rebuilt: [K][N] rows past the slice, and with wide steps
      // [N][K] columns past the slice (a slice of an odd number of 64-wide
      // steps ends half way through its last step).  Chunks past N only feed
      // output columns that are never stored.
      if constexpr (LAYOUT == 0) {
        wval[i] = KW == 1 || kstep + wkr < klen;
      } else {
        wval[i] = kstep + wkr + i * (NT / QN) < klen;
      }
    }
    if (part == 3) {   // the step's last part: every chunk of the step has loaded
      xo += 2u * BK;
      wo += wadv;
      kstep += BK;
    }
  };
  // registers of a step -> LDS buffer (x as is, weights rebuilt)
  auto store_step = [&](uint16_t* xs, uint16_t* ws, int part) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      if (!in_part(i, XC, part)) continue;
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&xs[((uint32_t)c / XPR) * LDK + ((uint32_t)c % XPR) * 8]) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      if (!in_part(i, WC, part)) continue;
      uint32_t o[8];
      rebuild_raw<FMT>(w, wr[i], wval[i], wverb[i], whi, o);
      const int c = tid + i * NT;
      uint4* d;
      if constexpr (LAYOUT == 0) {
        d = reinterpret_cast<uint4*>(&ws[((uint32_t)c / WPR) * LDK + ((uint32_t)c % WPR) * 16]);
      } else {
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
    if constexpr (!XREG) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8*>(&xs[row * LDK + kk + 8 * (lane >> 5)]);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (LAYOUT == 0) {
        const int col = wn * WN + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8*>(&ws[col * LDK + kk + 8 * (lane >> 5)]);
      } else {
        b[j] = b_frag_kmajor(ws, LDW, kk, wn * WN + j * 32, lane);
      }
    }
  };
  // the MFMAs of k slice sl; XREG takes A from the slice's registers, which
  // then load the slice four on
  auto mfma_set = [&](int sl, const bf16x8 (&a)[TM], const bf16x8 (&b)[TN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (XREG) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[sl % 4][i], b[j], acc[i][j], 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
      }
    if constexpr (XREG) {
      load_xa(sl % 4);
      if (sl % 4 == 3) xao += 4u * 1024u;
    }
  };

  uint16_t* const xs0 = lds;
  uint16_t* const xs1 = lds + XS;
  uint16_t* const ws0 = lds + 2 * XS;
  uint16_t* const ws1 = lds + 2 * XS + WS;

  // prologue: step 0 in LDS buffer 0, step 1 in registers, flags of step 2
  // loaded (XREG: x of step 0 in registers)
  if constexpr (XREG) {
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) load_xa(sl);
    xao += 4u * 1024u;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if constexpr (fmt_is_pal(FMT)) load_flags(p, false);
    load_step(p);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if constexpr (fmt_is_pal(FMT)) load_flags(p, false);
    store_step(xs0, ws0, p);
    load_step(p);
    if constexpr (fmt_is_pal(FMT)) load_flags(p, true);
  }

  // step s: MFMAs from buffer s & 1 while step s+1 is rebuilt into the other
  // buffer and the raw data of step s+2 is requested; one barrier per step.
  // The last steps rebuild and load past the K range (clamped, zeroed, never
  // read) instead of branching, so every part is one basic block.
  auto body = [&](int st, const uint16_t* xs_c, const uint16_t* ws_c, uint16_t* xs_n, uint16_t* ws_n) __attribute__((always_inline)) {
    __syncthreads();
    // part p: the MFMAs of k slice p (fragments read one part earlier), the
    // next slice's fragment reads, and a quarter of the next step's rebuild
    // and of the raw loads two steps ahead
    auto rest = [&](int p) __attribute__((always_inline)) {
      store_step(xs_n, ws_n, p);
      load_step(p);
      if constexpr (fmt_is_pal(FMT)) load_flags(p, true);
      // ask the scheduler to alternate one MFMA with a few VALU operations of
      // the rebuild, so the vector ALU works while the matrix core runs
#pragma unroll
      for (int q = 0; q < KW * TM * TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // k slice sl runs from fragment set sl % 2, which then reads slice
    // sl + 2; part p follows slice KW (p + 1) - 1
    read_frags(xs_c, ws_c, 0, fa0, fb0);
    read_frags(xs_c, ws_c, 16, fa1, fb1);
#pragma unroll
    for (int sl = 0; sl < 4 * KW; ++sl) {
      if (sl % 2 == 0) {
        mfma_set(sl, fa0, fb0);
      } else {
        mfma_set(sl, fa1, fb1);
      }
      if (sl % KW == KW - 1) rest(sl / KW);
      if (sl + 2 < 4 * KW) {
        if (sl % 2 == 0) {
          read_frags(xs_c, ws_c, 16 * (sl + 2), fa0, fb0);
        } else {
          read_frags(xs_c, ws_c, 16 * (sl + 2), fa1, fb1);
        }
      }
    }
  };
  // XREG: drain the prologue's loads here, once.  Otherwise the compiler's
  // wait-count merge of the loop entry (where the last loads issued are the
  // ones the first step's rebuild reads) with the back edge (where x of the
  // next step loads last) puts a wait for every load in flight at the top of
  // each step, which exposes the x reloads' full latency once per step.
  if constexpr (XREG) __builtin_amdgcn_s_waitcnt(0);
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

// Tiles of the big-tile kernel: BM x BN, waves in a WGM x (waves / WGM) grid.
struct Tile2 {
  int bm, bn, waves, wgm;
  bool xreg;   // x in registers, only the weight tile in LDS (single rebuild per 512 rows)
  int nk_kw;   // K step of 64 nk_kw; 2 only for stored [N][K] weights
};
// 32-row tiles (one MFMA row tile, four waves side by side) are for small
// batches; then 256x256 with eight waves (two per SIMD); then the
// single-rebuild tile, 512 rows x 128 columns, eight waves of 64 rows.  The
// next six are the 64x128, 128x128, 32x128, 32x256 and single-rebuild tiles
// with 128-wide K steps for stored [N][K] weights, and a 256-row
// single-rebuild tile (eight waves of 32 rows) with them: each step reads
// whole 128-byte lines of sign+mantissa bytes per row (a 64-wide step reads
// half a line per row and the other half a step later), for twice the LDS
// (one block per CU for the four-wave tiles).  The last four run eight
// waves of 32 x 32 to 64 x 64 on the 128x128, 128x256 and 64x128 tiles:
// the same LDS as their four-wave versions, which it limits to one block
// per CU, holds twice the waves, so twice the loads are in flight and one
// wave's rebuild issues beside the other's MFMAs on each SIMD.
constexpr Tile2 kTiles2[] = {
    {64, 128, 4, 2, false, 1},  {128, 128, 4, 2, false, 1}, {128, 256, 4, 2, false, 1}, {256, 128, 4, 2, false, 1},
    {256, 256, 4, 2, false, 1}, {32, 128, 4, 1, false, 1},  {32, 256, 4, 1, false, 1},  {256, 256, 8, 2, false, 1},
    {512, 128, 8, 8, true, 1},  {64, 128, 4, 2, false, 2},  {128, 128, 4, 2, false, 2}, {32, 128, 4, 1, false, 2},
    {32, 256, 4, 1, false, 2},  {512, 128, 8, 8, true, 2},  {256, 128, 8, 8, true, 2}, {128, 128, 8, 2, false, 2},
    {128, 256, 8, 2, false, 1}, {64, 128, 8, 2, false, 1},  {64, 128, 8, 2, false, 2}};
constexpr int kTileCount = (int)(sizeof(kTiles2) / sizeof(kTiles2[0]));
constexpr int kLateFirst = 9;   // the first tile numbered after the register-fed kernels
constexpr int tile_kw(int tile) { return kTiles2[tile].nk_kw; }

// the kernel of tile T for layout L (none: a wide-step tile for [K][N])
template <int L, int F, int T>
Mfma2Fn inst() {
  constexpr Tile2 t = kTiles2[T];
  if constexpr (L == 1 && t.nk_kw > 1) {
    return nullptr;
  } else {
    return k_mfma2<L, F, t.bm, t.bn, t.wgm, t.waves, t.xreg, t.nk_kw>;
  }
}

template <int L, int F>
Mfma2Fn pick(int tile) {
  static_assert(kTileCount == 19, "one case per tile");
  switch (tile) {
    case 0: return inst<L, F, 0>();
    case 1: return inst<L, F, 1>();
    case 2: return inst<L, F, 2>();
    case 3: return inst<L, F, 3>();
    case 4: return inst<L, F, 4>();
    case 5: return inst<L, F, 5>();
    case 6: return inst<L, F, 6>();
    case 7: return inst<L, F, 7>();
    case 8: return inst<L, F, 8>();
    case 9: return inst<L, F, 9>();
    case 10: return inst<L, F, 10>();
    case 11: return inst<L, F, 11>();
    case 12: return inst<L, F, 12>();
    case 13: return inst<L, F, 13>();
    case 14: return inst<L, F, 14>();
    case 15: return inst<L, F, 15>();
    case 16: return inst<L, F, 16>();
    case 17: return inst<L, F, 17>();
    case 18: return inst<L, F, 18>();
    default: return nullptr;
  }
}

}  // namespace
int mfma2_tile_count() { return kTileCount; }
int mfma2_late_first() { return kLateFirst; }
void mfma2_tile_dims(int tile, int* bm, int* bn) {
  *bm = kTiles2[tile].bm;
  *bn = kTiles2[tile].bn;
}
void mfma2_tile_shape(int tile, int* waves, int* wgm, bool* xreg, int* kw) {
  *waves = kTiles2[tile].waves;
  *wgm = kTiles2[tile].wgm;
  *xreg = kTiles2[tile].xreg;
  *kw = kTiles2[tile].nk_kw;
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
  const size_t ldk = (size_t)ld_k(t.nk_kw);
  const size_t wtile = layout == 0 ? (size_t)t.bn * ldk : (size_t)kBK * (size_t)(t.bn + 16);
  return 2 * ((t.xreg ? 0 : (size_t)t.bm * ldk) + wtile) * sizeof(uint16_t);
}
// blocks a CU holds at once: by LDS, and one for the eight-wave tiles (their
// registers fill the SIMDs at two waves each)
int64_t mfma2_blocks_per_cu(int layout, const Tile2& t) {
  const int64_t by_lds = (int64_t)(160 * 1024 / mfma2_lds_bytes(layout, t));
  const int64_t b = t.waves == 8 ? 1 : by_lds;
  return b > 0 ? b : 1;
}

int mfma2_slices(const WeightView& w, int64_t batch, int tile, int split_hint) {
  const Tile2 t = kTiles2[tile];
  const int64_t blocks = ((int64_t)w.n + t.bn - 1) / t.bn * ((batch + t.bm - 1) / t.bm);
  const int64_t cus = (int64_t)device_cus();
  const int64_t target = batch <= 64 ? (fmt_is_pal(w.fmt) ? 512 : 256) : t.bm >= 256 ? (cus * 7 + 7) / 8 : 256;
  // up to 64 rows, and for tiles of 256 rows and more at any batch, never
  // past the blocks the CUs hold at once (a second round of blocks runs on
  // a mostly idle chip: 8B gate, palette-direct, 64 rows, 64x128 tiles: 4
  // slices 40.6 us, 8 slices 47.7 us; 70B q+k+v grouped, 40 256x256 tiles
  // at 192 rows: 4 slices 90 us, 8 slices 107 us; 8B q+k+v, 48 tiles at 384
  // rows: 4 slices 52 us, 8 slices 66 us; at 1024 rows with 512x128 tiles,
  // 8B q+k+v 96 tiles: 4 slices 91 us, 2 slices 71 us; 70B q+k+v 160 tiles:
  // 2 slices 239 us, none 198 us)
  const int64_t per_cu = mfma2_blocks_per_cu((int)w.layout, t);
  // the wide-step tiles (one block per CU) never queue a second round
  const bool one_round = batch <= 64 || t.bm >= 256 || t.nk_kw > 1;
  const int64_t hold = one_round ? cus * (per_cu > 0 ? per_cu : 1) : INT64_MAX;
  int s = split_hint > 0 ? split_hint : 1;
  if (split_hint <= 0)
    while (blocks * s < target && blocks * s * 2 <= hold && (int64_t)w.k / (64 * (s * 2)) >= 8) s *= 2;
  // a [K][N] block reads rows [kb, ke) of every column through one buffer
  // resource: at least enough slices that a slice's rows stay under its span
  if (w.layout == 1)
    while ((((int64_t)w.k + 64 * s - 1) / (64 * s)) * 64 * (int64_t)w.n * 2 > (int64_t)kRecMax &&
           (int64_t)w.k / (64 * (s * 2)) >= 1)
      s *= 2;
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

// Whether a tile with 128-wide K steps is the default in place of its
// 64-wide version: its grid at one block per CU, K split as above, still
// covers seven eighths of the CUs, and every block's K range is at least
// 2048 (16 steps), so its two-step prologue stays small against the loop.
// Where either fails the 64-wide tile, two or three blocks per CU, is faster.
// BF16 weights (two bytes each) already read whole lines with 64-wide steps.
bool mfma2_wide_pays(const WeightView& w, int64_t batch, int tile) {
  const Tile2 t = kTiles2[tile];
  if (w.layout != 0 || t.nk_kw < 2 || w.fmt == kFmtBf16) return false;
  const int64_t blocks = ((int64_t)w.n + t.bn - 1) / t.bn * ((batch + t.bm - 1) / t.bm);
  const int s = mfma2_slices(w, batch, tile, 0);
  const int64_t bk = 64 * (int64_t)t.nk_kw;
  const int64_t kslice = (((int64_t)w.k + bk - 1) / bk + s - 1) / s * bk;
  return blocks * s * 8 >= (int64_t)device_cus() * 7 && kslice >= 2048;
}

// bytes of x packed into A fragments for a tile that keeps x in registers
static size_t packed_x_bytes(const Tile2& t, int64_t batch, uint64_t k) {
  if (!t.xreg) return 0;
  const uint64_t mtiles = (uint64_t)((batch + t.bm - 1) / t.bm);
  return (size_t)(mtiles * (uint64_t)t.bm / 32 * ((k + 15) / 16) * 1024u);
}

// partial floats: the K slices' partial rows, then (x-in-register tiles)
// the packed x, 256-byte aligned
size_t mfma2_partial_elems(const WeightView& w, int64_t batch, int tile, int split_hint) {
  const int s = mfma2_slices(w, batch, tile, split_hint);
  const size_t slices = s > 1 ? (size_t)s * (size_t)batch * (size_t)w.n : 0;
  const size_t px = packed_x_bytes(kTiles2[tile], batch, w.k);
  return px ? (slices + 63) / 64 * 64 + px / 4 : slices;
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
  const int64_t bk = 64 * (int64_t)t.nk_kw;   // k per step
  const int64_t steps = ((int64_t)w0.k + bk - 1) / bk;
  const int64_t kslice = ((steps + slices - 1) / slices) * bk;
  // every buffer resource the kernel builds spans at most kRecMax bytes:
  // x, a [N][K] block's rows, a [K][N] slice's rows, the verbatim section
  if ((uint64_t)batch * w0.k * 2 > kRecMax) return hipErrorNotSupported;
  for (int i = 0; i < grp.count; ++i) {
    const WeightView& wi = grp.w[i];
    const uint64_t span = wi.layout == 0 ? (uint64_t)t.bn * wi.k : (uint64_t)kslice * wi.n;
    if (span * 2 > kRecMax || wi.vexp_bytes > kRecMax) return hipErrorNotSupported;
  }
  const bool split = slices > 1;
  const size_t split_elems = split ? (size_t)slices * (size_t)batch * (size_t)ntot : 0;
  const size_t px = packed_x_bytes(t, batch, w0.k);
  if (px > kRecMax) return hipErrorNotSupported;
  const size_t px_off = px ? (split_elems + 63) / 64 * 64 : split_elems;   // floats
  if ((split || px) && (part == nullptr || part_elems < px_off + px / 4)) return hipErrorInvalidValue;
  const uint16_t* xk = x;   // what the kernel reads as x
  if (px) {
    uint4* packed = reinterpret_cast<uint4*>(part + px_off);
    const int64_t pieces = (int64_t)(px / 16);
    hipLaunchKernelGGL(k_pack_xa, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, x, (int)batch,
                       (int64_t)w0.k, (int64_t)((w0.k + 15) / 16), pieces, packed);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    xk = reinterpret_cast<const uint16_t*>(packed);
  }
  Mfma2Fn f;
  if (t.nk_kw > 1 && w0.layout != 0) return hipErrorNotSupported;
  if (w0.layout == 0) {
    f = fmt == kFmtBf16 ? pick<0, kFmtBf16>(tile) : fmt == kFmtExp ? pick<0, kFmtExp>(tile)
        : fmt == kFmtPal ? pick<0, kFmtPal>(tile) : pick<0, kFmtPalRun>(tile);
  } else {
    f = fmt == kFmtBf16 ? pick<1, kFmtBf16>(tile) : fmt == kFmtExp ? pick<1, kFmtExp>(tile)
        : fmt == kFmtPal ? pick<1, kFmtPal>(tile) : pick<1, kFmtPalRun>(tile);
  }
  if (f == nullptr) return hipErrorNotSupported;
  const size_t lds = mfma2_lds_bytes((int)w0.layout, t);
  {
    hipError_t e = allow_dynamic_lds((const void*)f, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)nblocks, 1, (unsigned)slices);
  kernel_event_before(s);
  hipLaunchKernelGGL(f, grid, dim3(64 * t.waves), lds, s, grp, xk, (int)batch, y, ldy, kslice, split ? part : nullptr,
                     (int64_t)ntot, mtiles);
  hipError_t e = hipGetLastError();
  kernel_event_after(s);
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
