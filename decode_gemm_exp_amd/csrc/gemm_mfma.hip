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
// Structure (256 threads, 4 waves in a WGM x WGN grid, tile BM x BN, K step 64):
//   * the x tile and the rebuilt weight tile live in LDS, double buffered;
//   * while the waves run the MFMAs of step s, every thread already holds in
//     registers the raw data of step s+1 (x rows and compressed weights), and
//     for the palette format the verbatim flag words of step s+2, so the
//     dependent side-section loads of verbatim groups never stall;
//   * each weight is rebuilt once per block (not once per wave) straight into
//     LDS: NK rows with 16-byte stores, KN rows transposed with 16-bit stores;
//   * waves read A and B fragments from LDS and issue v_mfma_f32_32x32x16_bf16;
//   * split K: grid.z slices of K write partial tiles to the workspace and a
//     fixed-order reduction adds them (deterministic).
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

template <int FMT>
__device__ __forceinline__ void load_raw(const WeightView& w, uint64_t el, bool valid, uint32_t flagword,
                                         uint32_t rankword, Raw& r) {
  if (!valid) {
    r.a = make_uint4(0, 0, 0, 0);
    r.b = make_uint4(0, 0, 0, 0);
    return;
  }
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
    const uint8_t* p = group_verbatim(flagword, g)
                           ? w.vexp + (uint64_t)group_rank(flagword, rankword, g) * 64 + (el & 63)
                           : w.pidx + ((el >> 1) & ~(uint64_t)15);
    r.b = *reinterpret_cast<const uint4*>(p);
  }
}

// Rebuild 16 weights (8 dwords of packed bf16) from a raw chunk.
template <int FMT>
__device__ __forceinline__ void rebuild_raw(const WeightView& w, const Raw& r, bool valid, bool verbatim, bool hi,
                                            uint32_t o[8]) {
  if (!valid) {   // outside the matrix: exact zeros (a K tail multiplies them by zero x)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0;
    return;
  }
  if constexpr (FMT == kFmtBf16) {
    o[0] = r.a.x; o[1] = r.a.y; o[2] = r.a.z; o[3] = r.a.w;
    o[4] = r.b.x; o[5] = r.b.y; o[6] = r.b.z; o[7] = r.b.w;
  } else if constexpr (FMT == kFmtExp) {
    rebuild16(r.a, r.b, o);
  } else {
    uint4 e = pal16(hi ? r.b.z : r.b.x, hi ? r.b.w : r.b.y, w.pal);
    if (verbatim) e = r.b;
    rebuild16(r.a, e, o);
  }
}

template <int LAYOUT, int FMT, int BM, int BN, int WGM>
__global__ __launch_bounds__(256) void k_mfma2(WeightView w, const uint16_t* __restrict__ x, int B,
                                               float* __restrict__ y, int64_t ldy, int64_t col0,
                                               int64_t kslice, float* __restrict__ part) {
  constexpr int WGN = 4 / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int XC = BM * 8 / 256;     // 16-byte x chunks per thread per step
  constexpr int WC = BN * 4 / 256;     // 16-weight chunks per thread per step
  static_assert(TM >= 1 && TN >= 1 && XC >= 1 && WC >= 1, "tile too small");
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  uint16_t* Xs = lds;                          // [2][BM * kLDK]
  uint16_t* Ws = lds + 2 * BM * kLDK;          // [2][BN * kLDK]  (row = n, column = k)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t N = (int64_t)w.n, K = (int64_t)w.k;
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
  const int64_t kb = (int64_t)blockIdx.z * kslice;
  const int64_t ke = kb + kslice < K ? kb + kslice : K;

  // chunk c of this thread (i-th): NK -> row r = c / 4, k sub-block q = c % 4;
  // KN -> k row kr = c / (BN/16), n sub-block q = c % (BN/16)
  auto chunk_el = [&](int i, int64_t k0, bool& valid) -> uint64_t {
    const int c = tid + i * 256;
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
  uint32_t fw_next[WC], rk_next[WC];   // palette: flag / rank words of the step after the loaded one

  auto load_flags = [&](int64_t k0, uint32_t* fw, uint32_t* rk) {
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      bool v;
      const uint64_t el = chunk_el(i, k0, v);
      const uint64_t g = el >> 6;
      fw[i] = v ? w.vflags[g >> 5] : 0u;
      rk[i] = v ? w.vrank[g >> 5] : 0u;
    }
  };
  auto load_step = [&](int64_t k0, const uint32_t* fw, const uint32_t* rk) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = tid + i * 256;
      const int64_t row = m0 + (c >> 3), kk = k0 + (c & 7) * 8;
      xr[i] = (row < B && kk < ke) ? *reinterpret_cast<const uint4*>(x + row * K + kk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      bool v;
      const uint64_t el = chunk_el(i, k0, v);
      load_raw<FMT>(w, el, v, fw[i], rk[i], wr[i]);
      wval[i] = v;
      wverb[i] = FMT == kFmtPal && v && group_verbatim(fw[i], el >> 6);
      whi[i] = (el & 16) != 0;
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint32_t fw_cur[WC], rk_cur[WC];
  if constexpr (FMT == kFmtPal) {
    load_flags(kb, fw_cur, rk_cur);
    load_flags(kb + kBK, fw_next, rk_next);
  } else {
#pragma unroll
    for (int i = 0; i < WC; ++i) fw_cur[i] = rk_cur[i] = fw_next[i] = rk_next[i] = 0;
  }
  load_step(kb, fw_cur, rk_cur);

  int buf = 0;
  for (int64_t k0 = kb; k0 < ke; k0 += kBK) {
    uint16_t* xs = Xs + buf * BM * kLDK;
    uint16_t* ws = Ws + buf * BN * kLDK;
    // ---- registers of step k0 -> LDS (x as is, weights rebuilt) ----
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<uint4*>(&xs[(c >> 3) * kLDK + (c & 7) * 8]) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      uint32_t o[8];
      rebuild_raw<FMT>(w, wr[i], wval[i], wverb[i], whi[i], o);
      const int c = tid + i * 256;
      if constexpr (LAYOUT == 0) {
        uint4* d = reinterpret_cast<uint4*>(&ws[(c >> 2) * kLDK + (c & 3) * 16]);
        d[0] = make_uint4(o[0], o[1], o[2], o[3]);
        d[1] = make_uint4(o[4], o[5], o[6], o[7]);
      } else {
        constexpr int QN = BN / 16;
        const int kr = c / QN, q = c % QN;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          ws[(q * 16 + e) * kLDK + kr] = (uint16_t)((o[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
    }
    // ---- raw data of the next step -> registers (latency hidden by the MFMAs) ----
    if (k0 + kBK < ke) {
      if constexpr (FMT == kFmtPal) {
#pragma unroll
        for (int i = 0; i < WC; ++i) {
          fw_cur[i] = fw_next[i];
          rk_cur[i] = rk_next[i];
        }
        load_step(k0 + kBK, fw_cur, rk_cur);
        if (k0 + 2 * kBK < ke) load_flags(k0 + 2 * kBK, fw_next, rk_next);
      } else {
        load_step(k0 + kBK, fw_cur, rk_cur);
      }
    }
    __syncthreads();
    // ---- MFMA over the step ----
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8*>(&xs[row * kLDK + kk + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = wn * WN + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8*>(&ws[col * kLDK + kk + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    buf ^= 1;
  }

  // ---- epilogue: y, or this K slice's partial tile part[slice][row][col] ----
  float* out = part ? part + (uint64_t)blockIdx.z * (uint64_t)B * (uint64_t)N : y + col0;
  const int64_t ld = part ? N : ldy;
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

typedef void (*Mfma2Fn)(WeightView, const uint16_t*, int, float*, int64_t, int64_t, int64_t, float*);

template <int L, int F, int BM, int BN, int WGM>
Mfma2Fn prepared() {
  static bool done = false;
  if (!done) {
    const int lds = (int)(2 * (BM + BN) * kLDK * sizeof(uint16_t));
    (void)hipFuncSetAttribute((const void*)k_mfma2<L, F, BM, BN, WGM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    done = true;
  }
  return k_mfma2<L, F, BM, BN, WGM>;
}

template <int L, int F>
Mfma2Fn pick(int tile) {
  switch (tile) {
    case 0: return prepared<L, F, 64, 128, 2>();
    case 1: return prepared<L, F, 128, 128, 2>();
    case 2: return prepared<L, F, 128, 256, 2>();
    case 3: return prepared<L, F, 256, 128, 2>();
    default: return prepared<L, F, 256, 256, 2>();
  }
}

}  // namespace

// Tiles of the big-tile kernel: {BM, BN}.
struct Tile2 {
  int bm, bn;
};
static const Tile2 kTiles2[] = {{64, 128}, {128, 128}, {128, 256}, {256, 128}, {256, 256}};
int mfma2_tile_count() { return (int)(sizeof(kTiles2) / sizeof(kTiles2[0])); }

// K slices so that the grid covers the chip at least once (capped; each slice >= 8 steps)
int mfma2_slices(const WeightView& w, int64_t batch, int tile, int split_hint) {
  const Tile2 t = kTiles2[tile];
  const int64_t blocks = ((int64_t)w.n + t.bn - 1) / t.bn * ((batch + t.bm - 1) / t.bm);
  int s = split_hint > 0 ? split_hint : 1;
  if (split_hint <= 0)
    while (blocks * s < 256 && (int64_t)w.k / (64 * (s * 2)) >= 8) s *= 2;
  const int64_t steps = ((int64_t)w.k + 63) / 64;
  if (s > steps) s = (int)steps;
  return s;
}

size_t mfma2_partial_elems(const WeightView& w, int64_t batch, int tile, int split_hint) {
  const int s = mfma2_slices(w, batch, tile, split_hint);
  return s > 1 ? (size_t)s * (size_t)batch * (size_t)w.n : 0;
}

hipError_t launch_mfma2(const WeightView& w, const uint16_t* x, int64_t batch, float* y, int64_t ldy, int64_t col0,
                        int tile, int split_hint, float* part, size_t part_elems, hipStream_t s) {
  const Tile2 t = kTiles2[tile];
  const int slices = mfma2_slices(w, batch, tile, split_hint);
  const int64_t steps = ((int64_t)w.k + 63) / 64;
  const int64_t kslice = ((steps + slices - 1) / slices) * 64;
  const bool split = slices > 1;
  if (split && (part == nullptr || part_elems < (size_t)slices * (size_t)batch * (size_t)w.n))
    return hipErrorInvalidValue;
  Mfma2Fn f;
  if (w.layout == 0) {
    f = w.fmt == kFmtBf16 ? pick<0, kFmtBf16>(tile) : w.fmt == kFmtExp ? pick<0, kFmtExp>(tile) : pick<0, kFmtPal>(tile);
  } else {
    f = w.fmt == kFmtBf16 ? pick<1, kFmtBf16>(tile) : w.fmt == kFmtExp ? pick<1, kFmtExp>(tile) : pick<1, kFmtPal>(tile);
  }
  const size_t lds = 2 * (size_t)(t.bm + t.bn) * kLDK * sizeof(uint16_t);
  dim3 grid((unsigned)((w.n + (uint64_t)t.bn - 1) / (uint64_t)t.bn), (unsigned)((batch + t.bm - 1) / t.bm),
            (unsigned)slices);
  hipLaunchKernelGGL(f, grid, dim3(256), lds, s, w, x, (int)batch, y, ldy, col0, kslice, split ? part : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  return launch_sum_slices(part, slices, w.n, batch, y, ldy, col0, s);
}

}  // namespace uw
