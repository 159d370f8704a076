// gemm.hip -- y = x . W^T from BF16, exponent+sign/mantissa, or palette+
// sign/mantissa weights, for stored W[N][K] (NK) or W^T[K][N] (KN).
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "重建矩陣乘法核心運作": the
// matmul loads compressed weights, rebuilds BF16 in on-chip memory and feeds
// the matrix units, so rebuilt weights never go back to HBM.  Section
// "四種執行管道": small batches are dominated by fixed costs, large batches
// by the matmul; section "未來方向": the down projection's transposed
// dimensions need their own kernel (the KN paths below).
//
// Two families:
//   * GEMV (batch <= 8 per launch): VALU, v_dot2_f32_bf16 on rebuilt pairs,
//     software-pipelined so that the loads of the next step are in flight
//     while the current one is rebuilt.  NK: a wave per output row, lanes
//     stride K in 16-weight chunks, wave reduction.  KN: lanes own 16
//     consecutive outputs, waves take row pairs, partial sums per K slice go
//     to the workspace and a second kernel adds them in a fixed order
//     (deterministic).
//   * MFMA: gemm_mfma.hip.
#include <cmath>
#include <cstring>

#include <cstdio>

#include "rebuild.h"

namespace uw {
namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// ---- GEMV, stored [N][K], K a multiple of 1024 U --------------------------------
// One block per CU of 8..16 waves (the host picks the count that spreads the
// rows most evenly over CUs), x rows staged once per block in LDS.
// A wave owns rows n = wave, wave + nwaves, ... and walks each in steps of
// 1024 U weights (lane: U chunks of 16 at lane * 16 + u * 1024).  Software
// pipeline over the wave's steps, two register buffers: while step j is
// rebuilt and multiplied, the chunks of step j+1 are in flight and the
// palette flag/rank words of steps j+2, j+3 too.  Row end: wave reduction.
//
// One launch can serve up to kGemvGroupMax matrices with the same K and x
// (fused q+k+v, gate+up): matrix i owns the waves [wave0[i], wave0[i+1]) and
// writes output columns col0[i] ..; a single matrix is a group of one.
// Small matrices give each wave only a step or two, so one launch instead
// of one per matrix saves the pipeline's fill and drain per matrix.
struct GemvGroup {
  WeightView w[kGemvGroupMax];
  int64_t col0[kGemvGroupMax];
  uint32_t wave0[kGemvGroupMax + 1];
  int count;
};

template <int FMT, int NB, int U>
__global__ __launch_bounds__(1024) void k_gemv_nk_pipe(GemvGroup grp, const uint16_t* __restrict__ x, int B,
                                                       float* __restrict__ y, int64_t ldy) {
  extern __shared__ uint4 xs4[];   // B rows of K bf16
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(xs4);
  const int lane = threadIdx.x & 63;
  const uint32_t wpb = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);   // keeps the wave math scalar
  const uint32_t gwave = blockIdx.x * wpb + wave_uniform(threadIdx.x >> 6);
  int gi = 0;
#pragma unroll
  for (int i = 1; i < kGemvGroupMax; ++i) gi += (i < grp.count && gwave >= grp.wave0[i]) ? 1 : 0;
  gi = (int)wave_uniform((uint32_t)gi);
  const WeightView w = grp.w[gi];
  const int64_t col0 = grp.col0[gi];
  const uint64_t K = w.k, N = w.n;
  const uint64_t wave = gwave - grp.wave0[gi];
  const uint64_t nw = grp.wave0[gi + 1] - grp.wave0[gi];
  const uint32_t spr = (uint32_t)(K / (1024u * U));         // steps per row
  const uint64_t steps = (gwave < grp.wave0[grp.count] && wave < N) ? ((N - 1 - wave) / nw + 1) * spr : 0u;
  // cursor of a step: row and part; advanced one step at a time
  struct Cur {
    uint64_t row;
    uint32_t part;
  };
  auto advance = [&](Cur& c) {
    if (++c.part == spr) {
      c.part = 0;
      c.row += nw;
    }
  };
  auto el_of = [&](const Cur& c, int u) -> uint64_t {
    return c.row * K + (uint64_t)c.part * (1024u * U) + (uint64_t)u * 1024u + (uint64_t)lane * 16u;
  };

  // The steady-state loop issues the same loads on every path, so the
  // compiler's wait counts are exact and step j's products wait only for
  // step j's data (loads behind branches made them wait for every load in
  // flight).  Load cursors stop at the wave's last step; a wave without
  // rows reads row 0 and leaves after the barrier.  The palette flag and rank words of a
  // step are the same for all lanes (lanes cover 1024 weights from a
  // 1024-aligned start, a flag word 2048), so with no global store before
  // them they are scalar loads and never wait behind the chunks: the row
  // sums stay in registers (lane i keeps the wave's i-th row, at most 64)
  // and go to y after the loop.
  ChunkT<16> da[U], db[U];
  uint32_t fa[U], ra[U], fb[U], rb[U];   // flag/rank words of the chunks in da / db
  uint32_t ga[U], gha[U], gb[U], ghb[U]; // flag/rank words of the next steps of each parity
  Cur cc{wave < N ? wave : 0u, 0};       // step being computed
  Cur cl = cc;                           // next step whose chunks get loaded
  Cur cf = cc;                           // next step whose flags get loaded
  uint64_t li = 0, fi = 0;               // step indices of cl and cf
  auto next = [&](Cur& c, uint64_t& i) {
    if (i + 1 < steps) {
      advance(c);
      ++i;
    }
  };
  auto load_flags = [&](uint32_t* f, uint32_t* r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (fmt_is_pal(FMT)) {
        const uint64_t fw = (cf.row * K + (uint64_t)cf.part * (1024u * U) + (uint64_t)u * 1024u) >> 11;
        f[u] = w.vflags[fw];
        r[u] = w.vrank[fw];
      } else {
        f[u] = r[u] = 0;
      }
    }
    next(cf, fi);
  };
  // live = false: the prologue's second step of a one-step wave; every lane
  // reads the matrix's first 16 bytes (one line) instead of a whole step
  auto load_chunks = [&](ChunkT<16>* d, const uint32_t* f, const uint32_t* r, bool live) {
#pragma unroll
    for (int u = 0; u < U; ++u) chunk_load<FMT, 16, true>(w, live ? el_of(cl, u) : 0u, live ? f[u] : 0u, r[u], d[u]);
    next(cl, li);
  };

  // The first two steps' loads go out before x is staged and the block
  // meets at the barrier, so their latency overlaps both.  Palette chunks
  // need their flag words for the address: flags first, chunks after the
  // x copy.
  load_flags(fa, ra);
  load_flags(fb, rb);
  if constexpr (!fmt_is_pal(FMT)) {
    load_chunks(da, fa, ra, true);
    load_chunks(db, fb, rb, steps > 1);
  }
  {
    const uint32_t pieces = (uint32_t)((uint64_t)B * K / 8);
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    for (uint32_t i = threadIdx.x; i < pieces; i += blockDim.x) xs4[i] = x4[i];
  }
  if constexpr (fmt_is_pal(FMT)) {
    load_chunks(da, fa, ra, true);
    load_chunks(db, fb, rb, steps > 1);
  }
  load_flags(ga, gha);
  load_flags(gb, ghb);
  __syncthreads();
  if (steps == 0) return;

  float acc[NB], res[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = res[b] = 0.f;
  uint32_t rows_done = 0;

  // products of the step at cc; at a row end lane rows_done keeps the sums
  auto compute = [&](const ChunkT<16>* d, const uint32_t* f) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t o[8];
      chunk_rebuild<FMT, 16>(w, d[u], el_of(cc, u), f[u], o);
      const uint64_t k = (uint64_t)cc.part * (1024u * U) + (uint64_t)u * 1024u + (uint64_t)lane * 16u;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < B) {
          const uint4* xp = reinterpret_cast<const uint4*>(xs + (uint64_t)b * K + k);
          const uint4 x0 = xp[0], x1 = xp[1];
          float a = acc[b];
          a = dot2(o[0], x0.x, a); a = dot2(o[1], x0.y, a);
          a = dot2(o[2], x0.z, a); a = dot2(o[3], x0.w, a);
          a = dot2(o[4], x1.x, a); a = dot2(o[5], x1.y, a);
          a = dot2(o[6], x1.z, a); a = dot2(o[7], x1.w, a);
          acc[b] = a;
        }
      }
    }
    if (cc.part == spr - 1) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float t = wave_sum(acc[b]);
        res[b] = (uint32_t)lane == rows_done ? t : res[b];
        acc[b] = 0.f;
      }
      ++rows_done;
    }
    advance(cc);
  };

  // steady state: da/db hold steps j, j+1 and the loads of j+2, j+3 all
  // exist; the last one to three steps run after the loop
  uint64_t j = 0;
  for (; j + 3 < steps; j += 2) {
    compute(da, fa);               // step j
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fa[u] = ga[u];
      ra[u] = gha[u];
    }
    load_chunks(da, fa, ra, true);   // step j+2
    load_flags(ga, gha);             // step j+4 (or the last)
    compute(db, fb);               // step j+1
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fb[u] = gb[u];
      rb[u] = ghb[u];
    }
    load_chunks(db, fb, rb, true);   // step j+3
    load_flags(gb, ghb);             // step j+5 (or the last)
  }
  compute(da, fa);                 // step j
  if (j + 2 < steps) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      fa[u] = ga[u];
      ra[u] = gha[u];
    }
    load_chunks(da, fa, ra, true);   // step j+2
  }
  if (j + 1 < steps) compute(db, fb);
  if (j + 2 < steps) compute(da, fa);
  // row i of this wave is wave + i * nw
  if ((uint32_t)lane < rows_done) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < B) y[(uint64_t)b * ldy + col0 + wave + (uint64_t)lane * nw] = res[b];
  }
}

// ---- GEMV, stored [N][K], any K (multiple of 16) ----------------------------------
// One wave per output row; each lane takes kGemvU chunks of 16 weights per
// pass (K positions lane*16 + u*1024), loads first, then the products.
constexpr int kGemvU = 4;

template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_gemv_nk_any(WeightView w, const uint16_t* __restrict__ x, int B,
                                                     float* __restrict__ y, int64_t ldy, int64_t col0) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave_id = ((uint64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const uint64_t nwaves = (uint64_t)gridDim.x * 4;
  const uint64_t K = w.k;
  for (uint64_t n = wave_id; n < w.n; n += nwaves) {
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    for (uint64_t k0 = (uint64_t)lane * 16; k0 < K; k0 += 1024 * kGemvU) {
      uint32_t wv[kGemvU][8];
#pragma unroll
      for (int u = 0; u < kGemvU; ++u) {
        const uint64_t k = k0 + (uint64_t)u * 1024;
        if (k < K) {
          load16<FMT>(w, n * K + k, wv[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) wv[u][i] = 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kGemvU; ++u) {
        const uint64_t k = k0 + (uint64_t)u * 1024;
        if (k >= K) break;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            const uint4* xp = reinterpret_cast<const uint4*>(x + (uint64_t)b * K + k);
            const uint4 x0 = xp[0], x1 = xp[1];
            float a = acc[b];
            a = dot2(wv[u][0], x0.x, a); a = dot2(wv[u][1], x0.y, a);
            a = dot2(wv[u][2], x0.z, a); a = dot2(wv[u][3], x0.w, a);
            a = dot2(wv[u][4], x1.x, a); a = dot2(wv[u][5], x1.y, a);
            a = dot2(wv[u][6], x1.z, a); a = dot2(wv[u][7], x1.w, a);
            acc[b] = a;
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float t = wave_sum(acc[b]);
      if (b < B && lane == 0) y[(uint64_t)b * ldy + col0 + n] = t;
    }
  }
}

// ---- GEMV, stored [K][N] -----------------------------------------------------------
// Blocks of 8 waves; grid.x: blocks of 64 OW columns (lane: OW = 16 or 8
// consecutive outputs), grid.y: K slices.  A wave takes row pairs (k, k+1) of its slice,
// pairs wave, wave + 8, ..., U pairs per pipeline step (same two-buffer
// pipeline as the NK kernel).  The two rows' rebuilt weights are interleaved
// per column so that one v_dot2 multiplies (w[k][n], w[k+1][n]) with
// (x[k], x[k+1]).  The slice of x is staged in LDS (zero past the slice), so
// the products never wait on a global load.  At the end the 8 waves' sums
// meet in LDS (fixed order) and the block writes one partial row per batch
// row: part[slice][b][n].
constexpr int kKnWaves = 8;
constexpr uint32_t kKnXLdsMax = 32u * 1024u;   // staged x bytes per block

// SF (palette formats, N a multiple of the block's 64 OW columns): the
// block's columns of a row lie in one 2048-weight flag word, so the flag and
// rank words are wave-uniform scalar loads and never wait behind the chunks.
template <int FMT, int NB, int U, int OW, bool SF>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(NB <= 4 ? 4 : 2))) void k_gemv_kn(WeightView w, const uint16_t* __restrict__ x, int B,
                                                 float* __restrict__ part, uint32_t pairs_per_slice) {
  constexpr int BW = 64 * OW;   // columns per block
  __shared__ float red[kKnWaves][BW];
  extern __shared__ uint32_t xs2[];   // [B][pairs_per_slice] x pairs of the slice
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_uniform(threadIdx.x >> 6);
  const uint64_t N = w.n, K = w.k;
  const uint64_t n = (uint64_t)blockIdx.x * BW + (uint64_t)lane * OW;
  const bool nval = n < N;
  const uint64_t ncl = nval ? n : 0;                     // loads of columns past N read column 0
  const uint64_t kb = (uint64_t)blockIdx.y * 2u * pairs_per_slice;
  const uint64_t ke = kb + 2u * (uint64_t)pairs_per_slice < K ? kb + 2u * (uint64_t)pairs_per_slice : K;
  const uint32_t pairs = kb < ke ? (uint32_t)((ke - kb + 1) / 2) : 0u;
  const uint32_t mine = pairs > wave ? (pairs - 1 - wave) / kKnWaves + 1 : 0u;
  const uint32_t steps = (mine + U - 1) / U;

  // row of chunk h (0, 1) of pair slot u in step j; rows past the slice are
  // clamped for addressing, their rebuilt weights are zeroed
  auto row_of = [&](uint32_t j, int u, int h) -> uint64_t {
    return kb + 2u * (uint64_t)(wave + kKnWaves * (j * U + (uint32_t)u)) + (uint64_t)h;
  };
  auto el_of = [&](uint64_t k) -> uint64_t { return (k < K ? k : K - 1) * N + ncl; };
  // loads of steps past the wave's last read its last step again
  auto clampj = [&](uint32_t j) -> uint32_t { return j < steps ? j : (steps > 0 ? steps - 1 : 0u); };

  ChunkT<OW> da[U][2], db[U][2];
  uint32_t fa[U][2], ra[U][2], fb[U][2], rb[U][2];
  uint32_t ga[U][2], gha[U][2], gb[U][2], ghb[U][2];

  auto load_flags = [&](uint32_t j, uint32_t (*f)[2], uint32_t (*r)[2]) {
    j = clampj(j);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (SF) {
          const uint64_t k = row_of(j, u, h);
          const uint64_t fw = ((k < K ? k : K - 1) * N + (uint64_t)blockIdx.x * BW) >> 11;
          f[u][h] = w.vflags[fw];
          r[u][h] = w.vrank[fw];
        } else {
          flags_load<FMT>(w, el_of(row_of(j, u, h)), f[u][h], r[u][h]);
        }
      }
  };
  auto load_chunks = [&](uint32_t j, ChunkT<OW> (*d)[2], uint32_t (*f)[2], uint32_t (*r)[2]) {
    j = clampj(j);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) chunk_load<FMT, OW, true>(w, el_of(row_of(j, u, h)), f[u][h], r[u][h], d[u][h]);
  };

  // The steady-state loop issues the same loads on every path, so the
  // compiler's wait counts are exact (as in the NK kernel); the first two
  // steps' loads go out before x is staged.
  load_flags(0, fa, ra);
  load_flags(1, fb, rb);
  load_chunks(0, da, fa, ra);
  load_chunks(1, db, fb, rb);
  {
    const uint32_t total = (uint32_t)B * pairs_per_slice;
    for (uint32_t i = threadIdx.x; i < total; i += 512u) {
      const uint32_t b = i / pairs_per_slice, q = i - b * pairs_per_slice;
      const uint64_t k = kb + 2u * (uint64_t)q;
      const uint16_t* xr = x + (uint64_t)b * K;
      const uint32_t lo = k < ke ? xr[k] : 0u, hi = k + 1 < ke ? xr[k + 1] : 0u;
      xs2[i] = lo | (hi << 16);
    }
  }
  load_flags(2, ga, gha);
  load_flags(3, gb, ghb);
  __syncthreads();

  float acc[NB][OW];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < OW; ++i) acc[b][i] = 0.f;

  auto compute = [&](uint32_t j, ChunkT<OW> (*d)[2], uint32_t (*f)[2]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t k = row_of(j, u, 0);
      uint32_t o0[OW / 2], o1[OW / 2];
      chunk_rebuild<FMT, OW>(w, d[u][0], el_of(k), f[u][0], o0);
      chunk_rebuild<FMT, OW>(w, d[u][1], el_of(k + 1), f[u][1], o1);
      // a row past the slice (clamped load) contributes nothing, even where
      // its clamped weights are not finite
      if (k + 1 >= ke) {
#pragma unroll
        for (int i = 0; i < OW / 2; ++i) {
          o1[i] = 0u;
          if (k >= ke) o0[i] = 0u;
        }
      }
      const uint32_t q = (uint32_t)((k - kb) / 2u);
      uint32_t xv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) xv[b] = (b < B && k < ke) ? xs2[(uint32_t)b * pairs_per_slice + q] : 0u;
#pragma unroll
      for (int i = 0; i < OW / 2; ++i) {
        const uint32_t plo = __builtin_amdgcn_perm(o1[i], o0[i], 0x05040100u);
        const uint32_t phi = __builtin_amdgcn_perm(o1[i], o0[i], 0x07060302u);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            acc[b][2 * i] = dot2(plo, xv[b], acc[b][2 * i]);
            acc[b][2 * i + 1] = dot2(phi, xv[b], acc[b][2 * i + 1]);
          }
        }
      }
    }
  };

  uint32_t j = 0;
  for (; j + 3 < steps; j += 2) {
    compute(j, da, fa);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        fa[u][h] = ga[u][h];
        ra[u][h] = gha[u][h];
      }
    load_chunks(j + 2, da, fa, ra);
    load_flags(j + 4, ga, gha);
    compute(j + 1, db, fb);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        fb[u][h] = gb[u][h];
        rb[u][h] = ghb[u][h];
      }
    load_chunks(j + 3, db, fb, rb);
    load_flags(j + 5, gb, ghb);
  }
  // the last one to three steps
  if (j < steps) compute(j, da, fa);
  if (j + 2 < steps) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        fa[u][h] = ga[u][h];
        ra[u][h] = gha[u][h];
      }
    load_chunks(j + 2, da, fa, ra);
  }
  if (j + 1 < steps) compute(j + 1, db, fb);
  if (j + 2 < steps) compute(j + 2, da, fa);

  // the block's waves, added in wave order, one batch row at a time
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= B) break;
    float4* mine4 = reinterpret_cast<float4*>(&red[wave][lane * OW]);
#pragma unroll
    for (int i = 0; i < OW / 4; ++i)
      mine4[i] = make_float4(acc[b][4 * i], acc[b][4 * i + 1], acc[b][4 * i + 2], acc[b][4 * i + 3]);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < BW / 512; ++h) {
      const uint32_t c = threadIdx.x + 512u * (uint32_t)h;
      float s = red[0][c];
#pragma unroll
      for (int v = 1; v < kKnWaves; ++v) s += red[v][c];
      const uint64_t col = (uint64_t)blockIdx.x * BW + c;
      if (col < N) part[((uint64_t)blockIdx.y * (uint64_t)B + (uint64_t)b) * N + col] = s;
    }
    __syncthreads();
  }
}

// y[b][col0 + n] = sum over slices p of part[p][b][n], four consecutive
// outputs per lane (N a multiple of 4): every slice is read with 16-byte
// loads, 1 KB per wave instruction, and added in slice order, so results
// repeat bit for bit.  The kernel below serves other N.
__global__ __launch_bounds__(256) void k_sum_slices4(const float4* __restrict__ part, int slices, uint64_t N4,
                                                     int64_t B, int64_t b0, float* __restrict__ y, int64_t ldy,
                                                     int64_t col0) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N4) return;
  const uint64_t b = (uint64_t)b0 + blockIdx.y;
  const uint64_t stride = (uint64_t)B * N4;
  const float4* src = part + b * N4 + i;
  float4 s = src[0];
  int p = 1;
  for (; p + 3 < slices; p += 4) {   // four loads in flight, added in order
    const float4 v0 = src[(uint64_t)p * stride], v1 = src[(uint64_t)(p + 1) * stride];
    const float4 v2 = src[(uint64_t)(p + 2) * stride], v3 = src[(uint64_t)(p + 3) * stride];
    s.x = (((s.x + v0.x) + v1.x) + v2.x) + v3.x;
    s.y = (((s.y + v0.y) + v1.y) + v2.y) + v3.y;
    s.z = (((s.z + v0.z) + v1.z) + v2.z) + v3.z;
    s.w = (((s.w + v0.w) + v1.w) + v2.w) + v3.w;
  }
  for (; p < slices; ++p) {
    const float4 v = src[(uint64_t)p * stride];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  float* dst = y + b * (uint64_t)ldy + (uint64_t)col0 + 4 * i;
  dst[0] = s.x;
  dst[1] = s.y;
  dst[2] = s.z;
  dst[3] = s.w;
}

// y[b][col0 + n] = sum over slices p of part[p][b][n].  Block: 4 waves on 64
// consecutive outputs of one batch row (grid.y = b); wave q adds slices
// q*L .. q*L+L-1 in order (loads batched 8 at a time), then the four wave
// sums are added in order q = 0..3 -- a fixed order, so results repeat
// bit for bit.
__global__ __launch_bounds__(256) void k_sum_slices(const float* __restrict__ part, int slices, uint64_t N,
                                                    int64_t B, int64_t b0, float* __restrict__ y, int64_t ldy,
                                                    int64_t col0) {
  __shared__ float sums[4][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const uint64_t n = (uint64_t)blockIdx.x * 64 + (uint64_t)lane;
  const uint64_t b = (uint64_t)b0 + blockIdx.y;
  const uint64_t stride = (uint64_t)B * N;
  const int L = (slices + 3) / 4;
  const int p0 = q * L, p1 = p0 + L < slices ? p0 + L : slices;
  float s = 0.f;
  if (n < N) {
    const float* src = part + b * N + n;
    for (int p = p0; p < p1; p += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p + u < p1 ? src[(uint64_t)(p + u) * stride] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (p + u < p1) s += v[u];
    }
  }
  sums[q][lane] = s;
  __syncthreads();
  if (q == 0 && n < N) y[b * (uint64_t)ldy + (uint64_t)col0 + n] = ((sums[0][lane] + sums[1][lane]) + sums[2][lane]) + sums[3][lane];
}

typedef void (*GemvNkFn)(WeightView, const uint16_t*, int, float*, int64_t, int64_t);
typedef void (*GemvPipeFn)(GemvGroup, const uint16_t*, int, float*, int64_t);
typedef void (*GemvKnFn)(WeightView, const uint16_t*, int, float*, uint32_t);

template <int F, int U>
GemvPipeFn gemv_nk_pipe_nb(int nb) {
  if (nb <= 1) return k_gemv_nk_pipe<F, 1, U>;
  if (nb <= 2) return k_gemv_nk_pipe<F, 2, U>;
  if (nb <= 4) return k_gemv_nk_pipe<F, 4, (U > 2 ? 2 : U)>;
  return k_gemv_nk_pipe<F, 8, (U > 2 ? 2 : U)>;
}
template <int F>
GemvPipeFn gemv_nk_pipe_fn(int nb, int u) {
  return u == 4 ? gemv_nk_pipe_nb<F, 4>(nb) : u == 2 ? gemv_nk_pipe_nb<F, 2>(nb) : gemv_nk_pipe_nb<F, 1>(nb);
}
template <int F>
GemvNkFn gemv_nk_any_fn(int nb) {
  if (nb <= 1) return k_gemv_nk_any<F, 1>;
  if (nb <= 2) return k_gemv_nk_any<F, 2>;
  if (nb <= 4) return k_gemv_nk_any<F, 4>;
  return k_gemv_nk_any<F, 8>;
}
// outputs per lane of the KN GEMV for a launch of nb batch rows
int kn_ow(int nb) { return nb <= 1 ? 16 : 8; }
template <int F, bool SF>
GemvKnFn gemv_kn_fn_sf(int nb) {
  if (nb <= 1) return k_gemv_kn<F, 1, 1, 16, SF>;
  if (nb <= 2) return k_gemv_kn<F, 2, 1, 8, SF>;
  if (nb <= 4) return k_gemv_kn<F, 4, 1, 8, SF>;
  return k_gemv_kn<F, 8, 1, 8, SF>;
}
// scalar flag loads for palette formats when N is a multiple of the block width
template <int F>
GemvKnFn gemv_kn_fn(int nb, uint64_t n) {
  if constexpr (fmt_is_pal(F)) {
    if (n % (64u * (uint64_t)kn_ow(nb)) == 0) return gemv_kn_fn_sf<F, true>(nb);
  }
  return gemv_kn_fn_sf<F, false>(nb);
}

constexpr int kGemvMaxBatch = 8;
constexpr uint64_t kGroupGemvMaxWeights = 96ull << 20;   // see launch_gemm_group
constexpr uint64_t kGroupTile32MaxWeights = 128ull << 20;   // see group_takes_tile32
constexpr size_t kNkLdsMax = 160 * 1024;


// chunks per lane per step of the pipelined NK GEMV (0: shape not covered)
int nk_pipe_u(const WeightView& w, int nb) {
  if ((uint64_t)nb * w.k * 2 > kNkLdsMax) return 0;
  if (w.k % 4096 == 0) return 4;
  if (w.k % 2048 == 0) return 2;
  if (w.k % 1024 == 0) return 1;
  return 0;
}

// Waves per block (8..16) and blocks (at most one per CU) of the pipelined
// NK GEMV.  Rows go to waves round-robin, so a CU's share is its waves times
// the most rows any wave gets; the count that makes the largest share
// smallest wins (ties: more waves).  Example: 14336 rows on 256 CUs take 14
// waves of 4 rows each, where 16 waves would leave half the CUs 64 rows and
// the other half 48.
int nk_pipe_waves(uint64_t n, uint64_t* blocks) {
  const uint64_t cus = (uint64_t)device_cus();
  int best = 16;
  uint64_t best_share = ~0ull;
  for (int wpb = 16; wpb >= 8; --wpb) {
    uint64_t g = (n + (uint64_t)wpb - 1) / (uint64_t)wpb;
    if (g > cus) g = cus;
    const uint64_t per_wave = (n + g * wpb - 1) / (g * wpb);
    const uint64_t share = per_wave * (uint64_t)wpb;
    if (share < best_share) {
      best_share = share;
      best = wpb;
    }
  }
  uint64_t g = (n + (uint64_t)best - 1) / (uint64_t)best;
  if (g > cus) g = cus;
  *blocks = g;
  return best;
}

// K slices of the KN GEMV: about two 8-wave blocks per CU over the grid,
// each wave with at least two pipeline steps of row pairs.
int kn_slices(const WeightView& w, int nb, const uw_kernel_cfg* cfg) {
  const uint64_t pairs = (w.k + 1) / 2;
  uint64_t s;
  if (cfg && cfg->split_k > 0) {
    s = (uint64_t)cfg->split_k;
  } else {
    const uint64_t bw = 64u * (uint64_t)kn_ow(nb);
    const uint64_t nblocks = (w.n + bw - 1) / bw;
    const uint64_t target = 2 * (uint64_t)device_cus();
    s = (target + nblocks - 1) / nblocks;
    const uint64_t max_s = pairs / (kKnWaves * 4);
    if (s > max_s) s = max_s;
  }
  // enough slices that a slice's x pairs fit the block's LDS stage
  const uint64_t per_slice_max = kKnXLdsMax / (4u * (uint64_t)(nb > 0 ? nb : 1));
  const uint64_t s_min = (pairs + per_slice_max - 1) / per_slice_max;
  if (s < s_min) s = s_min;
  if (s > pairs) s = pairs;
  if (s < 1) s = 1;
  return (int)s;
}

// Waves of a group launch: (blocks, waves per block) as for one matrix of
// all the group's rows, then each matrix gets waves in proportion to its
// rows (at least one, at most one per row).  False when the pipelined
// kernel cannot run the group: K not a multiple of 1024, x too large for
// LDS, or a wave left with more than 64 rows (one lane keeps each row's sum).
bool gemv_group_plan(GemvGroup& g, int nb, uint64_t* blocks, int* wpb) {
  if (nk_pipe_u(g.w[0], nb) == 0) return false;
  uint64_t total = 0;
  for (int i = 0; i < g.count; ++i) total += g.w[i].n;
  *wpb = nk_pipe_waves(total, blocks);
  const uint64_t T = *blocks * (uint64_t)*wpb;
  uint64_t wv[kGemvGroupMax] = {0, 0, 0, 0}, sum = 0;
  for (int i = 0; i < g.count; ++i) {
    uint64_t c = (T * g.w[i].n + total / 2) / total;
    if (c < 1) c = 1;
    if (c > g.w[i].n) c = g.w[i].n;
    wv[i] = c;
    sum += c;
  }
  while (sum > T) {   // rounding up the small ones: take the excess from the largest share
    int big = 0;
    for (int i = 1; i < g.count; ++i)
      if (wv[i] > wv[big]) big = i;
    if (wv[big] <= 1) return false;
    --wv[big];
    --sum;
  }
  g.wave0[0] = 0;
  for (int i = 0; i < g.count; ++i) {
    if ((g.w[i].n + wv[i] - 1) / wv[i] > 64) return false;
    g.wave0[i + 1] = g.wave0[i] + (uint32_t)wv[i];
  }
  for (int i = g.count + 1; i <= kGemvGroupMax; ++i) g.wave0[i] = g.wave0[g.count];
  return true;
}

// fmt: the weight format all matrices of the group are run in
hipError_t launch_gemv_group(const GemvGroup& g, int fmt, const uint16_t* x, int nb, float* y, int64_t ldy,
                             uint64_t blocks, int wpb, hipStream_t s) {
  const int u = nk_pipe_u(g.w[0], nb);
  GemvPipeFn f = fmt == kFmtBf16 ? gemv_nk_pipe_fn<kFmtBf16>(nb, u)
                 : fmt == kFmtExp ? gemv_nk_pipe_fn<kFmtExp>(nb, u)
                 : fmt == kFmtPal ? gemv_nk_pipe_fn<kFmtPal>(nb, u) : gemv_nk_pipe_fn<kFmtPalRun>(nb, u);
  hipError_t e = allow_dynamic_lds((const void*)f, (int)kNkLdsMax);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)nb * g.w[0].k * 2;
  hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(64 * wpb), lds, s, g, x, nb, y, ldy);
  return hipGetLastError();
}

}  // namespace

// Variant numbering seen through uw_kernel_cfg.variant: 1 = VALU GEMV (any
// batch, eight rows per launch), 2.. = the first nine MFMA tiles of
// gemm_mfma.hip (64-wide K steps), then the register-fed MFMA kernels of
// gemm_rf.hip, then the later tiles: those with 128-wide K steps (like the
// register-fed kernels, stored [N][K] only) and the eight-wave 128x128,
// 128x256 and 64x128 tiles.
int rf_first_variant() { return 2 + mfma2_late_first(); }
static int late_first_variant() { return rf_first_variant() + mfma_rf_kinds(); }
int gemm_variant_count() { return 1 + mfma2_tile_count() + mfma_rf_kinds(); }
bool gemm_variant_supported(int v, int layout) {
  if (layout == 0 || v < rf_first_variant()) return true;
  const int tile = gemm_variant_tile(v);   // none for the register-fed kernels
  if (tile < 0) return false;
  int waves = 0, wgm = 0, kw = 0;
  bool xreg = false;
  mfma2_tile_shape(tile, &waves, &wgm, &xreg, &kw);
  return kw == 1;
}
bool gemm_variant_is_rf(int v) { return v >= rf_first_variant() && v < late_first_variant(); }
int gemm_variant_tile(int v) {
  if (v >= 2 && v < rf_first_variant()) return v - 2;
  if (v >= late_first_variant() && v <= gemm_variant_count()) return mfma2_late_first() + (v - late_first_variant());
  return -1;
}
static int tile_variant(int tile) {
  return tile < mfma2_late_first() ? 2 + tile : late_first_variant() + (tile - mfma2_late_first());
}
// the wide-step versions of the 32x128 and single-rebuild tiles
static int wide_tile_32x128() { return mfma2_late_first() + 2; }
static int wide_tile_xreg() { return mfma2_late_first() + 4; }
static int wide_tile_xreg256() { return mfma2_late_first() + 5; }
// the eight-wave tiles: 128x128 and 64x128 with 128-wide K steps, 128x256
// with 64-wide ones (either layout)
static int eight_wave_128x128_wide() { return mfma2_late_first() + 6; }
static int eight_wave_128x256() { return mfma2_late_first() + 7; }
static int eight_wave_64x128_wide() { return mfma2_late_first() + 9; }

// Default kernel by batch, from sweeps over the 8B and 70B MLP shapes (every
// variant, both layouts, palette-direct and BF16 weights):
//   stored [N][K]: VALU GEMV up to 4 rows, register-fed MFMA up to 32 (x
//     shared through LDS, one row tile per wave, when its 64-row blocks
//     cover seven eighths of the CUs: 70B gate, palette, 8 / 16 / 32 rows
//     99.8 / 95.0 / 108.4 -> 84.6 / 83.5 / 96.7 us, 8B gate 8 / 16 rows 34.2
//     / 36.1 -> 31.6 / 32.1 us; on narrower matrices it loses, 8B q with 64
//     blocks at 8 rows 20.5 vs 13.2 us, and x per wave with two row tiles
//     per wave stays), then LDS tiles 64x128 up to 64, 128x128 up to 128
//     (both with eight waves and 128-wide K steps where those pay), the
//     eight-wave 256x256 up to 512 (K split to fill the CUs: 70B gate at
//     512 rows, palette-direct 466 -> 319 us, BF16 295 -> 234 us), and beyond
//     256x256 when its tiles cover seven eighths of the CUs (8B gate at 1024
//     rows, 224 tiles: palette-direct 252 -> 164 us), else 128x128 (8B q at
//     1024 rows, 64 tiles: 80 vs 81 us palette-direct, 46 vs 64 us BF16);
//   stored [K][N]: VALU GEMV for one row, then LDS tiles 32x256 up to 32,
//     the eight-wave 128x256 up to 128 (70B down, palette-direct, against
//     the four-wave 64x128 at 48 / 64 rows and 128x256 at 96 / 128 rows:
//     93.5 / 98.1 / 99.9 / 102.6 -> 84.8 / 89.2 / 91.7 / 101.1 us; on
//     another box 64 / 128 rows against 128x256 105.8 / 124.8 -> 99.4 /
//     102.7 us), 256x256 beyond (70B down at 192 rows, palette-direct: 292
//     -> 186 us).
// The 256x256 tile runs with eight waves (two per SIMD) for palette weights,
// whose rebuild then issues beside the other wave's MFMAs (70B gate,
// palette-direct, 1024 rows: 737 -> 602 us); BF16 and exponent weights gain
// nothing from it.  Tile indices are those of gemm_mfma.hip; tile_variant
// gives the variant number of a tile.
static int resolve_variant(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg) {
  if (cfg && cfg->variant > 0 && cfg->variant <= gemm_variant_count()) return cfg->variant;
  const int big = fmt_is_pal(w.fmt) ? 2 + 7 : 2 + 4;
  // the single-rebuild 512x128 tile (x in registers) beyond 256 rows when it
  // pads no more rows than 256-row tiles (an even number of 256-row tiles):
  // 70B at 1024 rows, palette-direct gate 507 -> 477 us, down 502 -> 457 us,
  // exponent gate 471 -> 435 us; at 512 rows palette-direct 267 -> 244 us
  // With stored [N][K] byte-format weights its 128-wide K steps read whole
  // lines per row (70B gate, palette-direct: 512 rows 240.5 -> 225.2 us,
  // 768 rows 430.4 -> 415.6, 1024 rows 449.3 -> 434.7, 2048 rows 879.9 ->
  // 851.4; exponent weights 1 % faster), identical results.
  if (batch > 256 && ((batch + 255) / 256) % 2 == 0)
    return w.layout == 0 && w.fmt != kFmtBf16 ? tile_variant(wide_tile_xreg()) : 2 + 8;
  if (w.layout == 0) {
    if (batch <= 4) return 1;
    if (batch <= 32 && mfma_rf_supported(w, 2) && (int64_t)((w.n + 63) / 64) * 8 >= (int64_t)device_cus() * 7)
      return rf_first_variant() + 2;
    if (batch <= 32 && mfma_rf_supported(w, 0)) return rf_first_variant();
    // 33 to 64 rows: the eight-wave 64x128 tile with 128-wide K steps where
    // those pay (70B gate, palette-direct, 48 / 64 rows: 110.0 / 103.5 us
    // against 114.1 / 111.7 for the register-fed kernel below and 117.1 /
    // 120.0 for the four-wave 64x128 tile); else x shared, two row tiles
    // per wave, when its 128-row
    // blocks cover seven eighths of the CUs (70B gate, palette, 40 / 48 / 64
    // rows: 115.4 / 110.9 / 113.5 us against 119.0 / 119.8 / 123.9 for the
    // 64x128 tile); narrower matrices keep the tile (8B gate 42.5 vs 38.1 us
    // at 64 rows)
    if (batch <= 64 && mfma2_wide_pays(w, batch, eight_wave_64x128_wide())) return tile_variant(eight_wave_64x128_wide());
    if (batch <= 64 && mfma_rf_supported(w, 3) && (int64_t)((w.n + 127) / 128) * 8 >= (int64_t)device_cus() * 7)
      return rf_first_variant() + 3;
    if (batch <= 64) return 2 + 0;
    // 65 to 128 rows: 128x128 tiles, eight waves with 128-wide K steps where
    // those pay (70B gate, palette-direct, against four waves: 96 / 128 rows
    // 110.6 / 108.7 -> 110.1 / 109.4 us on one box, 128 rows 127.9 -> 119.3
    // on another)
    if (batch <= 128)
      return mfma2_wide_pays(w, batch, eight_wave_128x128_wide()) ? tile_variant(eight_wave_128x128_wide()) : 2 + 1;
    // 129 to 256 rows: 256-row tiles; for byte-format weights the 256x128
    // single-rebuild tile with 128-wide K steps where those pay (70B gate,
    // palette-direct: 192 rows 159.2 -> 146.5 us, 256 rows 159.6 -> 152.5;
    // exponent weights at 256 rows 167.0 -> 152.4)
    if (batch <= 256 && mfma2_wide_pays(w, batch, wide_tile_xreg256())) return tile_variant(wide_tile_xreg256());
    if (batch <= 512) return 2 + 7;
    const int64_t tiles = (int64_t)((w.n + 255) / 256) * ((batch + 255) / 256);
    return tiles * 8 >= (int64_t)device_cus() * 7 ? big : 2 + 1;
  }
  if (batch == 1) return 1;
  if (batch <= 32) return 2 + 6;
  if (batch <= 128) return tile_variant(eight_wave_128x256());
  return big;
}

// The kernel one matrix call runs (uw_plan_gemm): variant, tile, K slices and
// the kernel's name as a profiler shows it (template arguments for the MFMA
// kernels, the family name for the GEMVs).
void describe_gemm(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg, uw_gemm_plan* out) {
  const int v = resolve_variant(w, batch, cfg);
  out->variant = v;
  out->fmt = w.fmt;
  out->tile_m = out->tile_n = out->waves = 0;
  out->k_slices = 1;
  if (v == 1) {
    const int nb = (int)(batch < kGemvMaxBatch ? batch : kGemvMaxBatch);
    if (w.layout == 0) {
      GemvGroup grp;
      std::memset(&grp, 0, sizeof(grp));
      grp.w[0] = w;
      grp.count = 1;
      uint64_t blocks = 0;
      int wpb = 0;
      const bool pipe = gemv_group_plan(grp, nb, &blocks, &wpb);
      std::snprintf(out->kernel, sizeof(out->kernel), "%s<%d, %d", pipe ? "k_gemv_nk_pipe" : "k_gemv_nk_any",
                    w.fmt, nb);
      out->waves = pipe ? wpb : 4;
    } else {
      out->k_slices = kn_slices(w, nb, cfg);
      std::snprintf(out->kernel, sizeof(out->kernel), "k_gemv_kn<%d, ", w.fmt);
      out->waves = 8;
    }
    return;
  }
  if (gemm_variant_is_rf(v)) {
    const int kind = v - rf_first_variant();
    const int tiles = kind == 0 ? 2 : kind == 1 ? 4 : kind == 2 ? 1 : 2;   // row tiles per wave
    out->tile_n = 16 * tiles;                                               // rows of W per wave
    out->tile_m = 16;
    out->waves = 4;
    out->k_slices = mfma_rf_slices(w, kind, cfg ? cfg->split_k : 0, device_cus());
    std::snprintf(out->kernel, sizeof(out->kernel), kind < 2 ? "k_mfma_rf<%d, %d, " : "k_mfma_rfx<%d, %d, ", w.fmt,
                  tiles);
    return;
  }
  const int tile = gemm_variant_tile(v);
  int bm = 0, bn = 0, waves = 0, wgm = 0, kw = 0;
  bool xreg = false;
  mfma2_tile_dims(tile, &bm, &bn);
  mfma2_tile_shape(tile, &waves, &wgm, &xreg, &kw);
  out->tile_m = bm;
  out->tile_n = bn;
  out->waves = waves;
  out->k_slices = mfma2_slices(w, batch, tile, cfg ? cfg->split_k : 0);
  std::snprintf(out->kernel, sizeof(out->kernel), "k_mfma2<%d, %d, %d, %d, %d, %d, %s, %d>", w.layout, w.fmt, bm, bn,
                wgm, waves, xreg ? "true" : "false", kw);
}

// From 8 to 32 rows a group of stored [N][K] matrices of at most 128 M
// weights runs as one launch of 32x128 LDS tiles over the whole group
// (unless a variant is forced).  Alone, each matrix would take the grouped
// GEMV (8 rows) or the register-fed kernel, launched once per matrix, and
// small matrices leave most of the chip idle in those launches.  Direct
// palette, default vs the 32-row group tile: 8B q+k+v at 8 / 16 / 32 rows
// 18.3 / 39.0 / 42.2 -> 16.6 / 17.0 / 18.1 us; 70B q+k+v 48.7 / 61.3 / 67.2
// -> 43.9 / 44.9 / 47.5 us; 8B gate+up 65.1 / 69.8 / 78.1 -> 55.6 / 57.4 /
// ~56 us.  The 70B gate+up pair (470 M weights) fills the chip matrix by
// matrix and gains nothing at 8 and 16 rows.  At 4 rows the grouped GEMV
// stays faster.
static bool group_takes_tile32(const WeightView* ws, int count, int64_t batch, const uw_kernel_cfg* cfg) {
  if (count < 2 || count > kMfma2GroupMax || batch < 8 || batch > 32 || (cfg && cfg->variant > 0)) return false;
  uint64_t total = 0;
  for (int i = 0; i < count; ++i) {
    if (ws[i].layout != 0 || ws[i].k != ws[0].k) return false;
    total += ws[i].n * ws[i].k;
  }
  return total <= kGroupTile32MaxWeights;
}

// One launch for a group of stored [N][K] matrices with the same K and x
// whose calls resolve to the VALU GEMV: output columns col0s[i] .. of y.
// hipErrorNotSupported when the group does not qualify (the caller then
// launches the matrices one by one).  Palette matrices of both kinds run
// with the general lookup unless all palettes are runs.
hipError_t launch_gemm_group(const WeightView* ws, int count, const uint16_t* x, int64_t batch, float* y,
                             int64_t ldy, const int64_t* col0s, const uw_kernel_cfg* cfg, hipStream_t s) {
  if (count < 2 || count > kGemvGroupMax || batch <= 0) return hipErrorNotSupported;
  if (group_takes_tile32(ws, count, batch, cfg)) return hipErrorNotSupported;
  const bool pal = fmt_is_pal(ws[0].fmt);
  // Up to 8 rows a group of small matrices takes the grouped GEMV even where
  // each matrix alone would take the register-fed kernel: one launch instead
  // of one per matrix (8B q+k+v, 25 M weights, 8 rows: 32.2 -> 18.9 us; 70B
  // q+k+v, 84 M: 52.5 -> 48.3 us).  Larger groups keep the per-matrix choice
  // (8B gate+up, 117 M: 63 us per-matrix against ~75 us grouped).
  uint64_t total = 0;
  for (int i = 0; i < count; ++i) total += ws[i].n * ws[i].k;
  const bool small_group = batch <= kGemvMaxBatch && total <= kGroupGemvMaxWeights && !(cfg && cfg->variant > 0);
  bool all_run = true;
  for (int i = 0; i < count; ++i) {
    if (ws[i].layout != 0 || ws[i].k != ws[0].k) return hipErrorNotSupported;
    if (!small_group && resolve_variant(ws[i], batch, cfg) != 1) return hipErrorNotSupported;
    if (fmt_is_pal(ws[i].fmt) != pal || (!pal && ws[i].fmt != ws[0].fmt)) return hipErrorNotSupported;
    all_run = all_run && ws[i].fmt == kFmtPalRun;
  }
  const int fmt = pal ? (all_run ? kFmtPalRun : kFmtPal) : ws[0].fmt;
  GemvGroup grp;
  std::memset(&grp, 0, sizeof(grp));
  grp.count = count;
  for (int i = 0; i < count; ++i) {
    grp.w[i] = ws[i];
    grp.col0[i] = col0s[i];
  }
  // the plan does not depend on the batch chunk beyond the LDS check of the largest one
  const int nb_max = (int)(batch < kGemvMaxBatch ? batch : kGemvMaxBatch);
  uint64_t blocks = 0;
  int wpb = 0;
  if (!gemv_group_plan(grp, nb_max, &blocks, &wpb)) return hipErrorNotSupported;
  for (int64_t b0 = 0; b0 < batch; b0 += kGemvMaxBatch) {
    const int nb = (int)(batch - b0 < kGemvMaxBatch ? batch - b0 : kGemvMaxBatch);
    hipError_t e = launch_gemv_group(grp, fmt, x + (uint64_t)b0 * ws[0].k, nb, y + (uint64_t)b0 * (uint64_t)ldy, ldy,
                                     blocks, wpb, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Workspace floats for partial sums of the kernel this call resolves to (the
// KN GEMV's K slices or the MFMA split-K slices).
size_t gemm_partial_elems(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg) {
  const int v = resolve_variant(w, batch, cfg);
  if (v == 1) {
    if (w.layout == 0) return 0;
    const int64_t rows = batch < kGemvMaxBatch ? batch : kGemvMaxBatch;
    return (size_t)kn_slices(w, (int)rows, cfg) * (size_t)rows * (size_t)w.n;
  }
  if (gemm_variant_is_rf(v))
    return w.layout == 0 ? mfma_rf_partial_elems(w, batch, v - rf_first_variant(), cfg ? cfg->split_k : 0,
                                                 device_cus())
                         : 0;
  return mfma2_partial_elems(w, batch, gemm_variant_tile(v), cfg ? cfg->split_k : 0);
}

// The most any variant needs at this batch (split hint as given).
size_t gemm_partial_elems_max(const WeightView& w, int64_t batch, int split_k) {
  uw_kernel_cfg c;
  c.variant = 0;
  c.split_k = split_k;
  c.decode_cus = 0;
  c.reserved = 0;
  size_t need = 0;
  for (int v = 1; v <= gemm_variant_count(); ++v) {
    c.variant = v;
    const size_t e = gemm_partial_elems(w, batch, &c);
    if (e > need) need = e;
  }
  return need;
}

hipError_t launch_sum_slices(const float* part, int slices, uint64_t n, int64_t batch, float* y, int64_t ldy,
                             int64_t col0, hipStream_t s) {
  const bool vec = n % 4 == 0 && (reinterpret_cast<uintptr_t>(part) & 15u) == 0;
  for (int64_t b0 = 0; b0 < batch; b0 += 65535) {
    const int64_t nb = batch - b0 < 65535 ? batch - b0 : 65535;
    if (vec)
      hipLaunchKernelGGL(k_sum_slices4, dim3((unsigned)((n / 4 + 255) / 256), (unsigned)nb), dim3(256), 0, s,
                         reinterpret_cast<const float4*>(part), slices, n / 4, batch, b0, y, ldy, col0);
    else
      hipLaunchKernelGGL(k_sum_slices, dim3((unsigned)((n + 63) / 64), (unsigned)nb), dim3(256), 0, s, part,
                         slices, n, batch, b0, y, ldy, col0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// A group (2..4 matrices of one layout, K and format class) that fits one
// LDS-tiled launch: the tile is the default (or forced) one of a matrix as
// wide as the group.  Returns the tile index, or -1.
static int tile_group_plan(const WeightView* ws, int count, int64_t batch, const uw_kernel_cfg* cfg) {
  if (count < 2 || count > kMfma2GroupMax || batch <= 0) return -1;
  WeightView wide = ws[0];
  uint64_t ntot = 0;
  for (int i = 0; i < count; ++i) {
    if (ws[i].layout != ws[0].layout || ws[i].k != ws[0].k) return -1;
    if (fmt_is_pal(ws[i].fmt) != fmt_is_pal(ws[0].fmt) || (!fmt_is_pal(ws[0].fmt) && ws[i].fmt != ws[0].fmt)) return -1;
    if (ws[i].fmt != ws[0].fmt) wide.fmt = kFmtPal;
    ntot += ws[i].n;
  }
  wide.n = ntot;
  if (group_takes_tile32(ws, count, batch, cfg))   // the 32x128 tile, with 128-wide K steps where those pay
    return mfma2_wide_pays(wide, batch, wide_tile_32x128()) ? wide_tile_32x128() : 5;
  const int v = resolve_variant(wide, batch, cfg);
  if (gemm_variant_tile(v) >= 0) return gemm_variant_tile(v);
  // The group as one matrix would take a register-fed kernel, which the
  // default picks by width.  From 33 to 64 rows the group is one launch of
  // 64x128 tiles instead (70B gate+up at 64 rows: 219.7 us against 228.9 us
  // matrix by matrix with the register-fed kernel; 8B gate+up, whose
  // matrices alone each take the tile: 63 us against 2 x 38 us).  Up to 32
  // rows it is one launch of the tile a matrix alone would take, if any;
  // matrices that each take the register-fed kernel run one by one.
  if (gemm_variant_is_rf(v) && !(cfg && cfg->variant > 0)) {
    if (batch > 32) return 0;
    for (int i = 0; i < count; ++i) {
      const int ti = gemm_variant_tile(resolve_variant(ws[i], batch, cfg));
      if (ti >= 0) return ti;
    }
  }
  return -1;
}

size_t gemm_tile_group_partial_elems(const WeightView* ws, int count, int64_t batch, const uw_kernel_cfg* cfg) {
  const int tile = tile_group_plan(ws, count, batch, cfg);
  if (tile < 0) return SIZE_MAX;
  return mfma2_group_partial_elems(ws, count, batch, tile, cfg ? cfg->split_k : 0);
}

hipError_t launch_gemm_tile_group(const WeightView* ws, int count, const uint16_t* x, int64_t batch, float* y,
                                  int64_t ldy, const int64_t* col0s, const uw_kernel_cfg* cfg, float* part,
                                  size_t part_elems, hipStream_t s) {
  const int tile = tile_group_plan(ws, count, batch, cfg);
  if (tile < 0) return hipErrorNotSupported;
  return launch_mfma2_group(ws, count, x, batch, y, ldy, col0s, tile, cfg ? cfg->split_k : 0, part, part_elems, s);
}

hipError_t launch_gemm(const WeightView& w, const uint16_t* x, int64_t batch, float* y, int64_t ldy,
                       int64_t col0, const uw_kernel_cfg* cfg, float* partial, size_t partial_elems,
                       hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  const int v = resolve_variant(w, batch, cfg);
  if (v == 1) {
    for (int64_t b0 = 0; b0 < batch; b0 += kGemvMaxBatch) {
      const int nb = (int)(batch - b0 < kGemvMaxBatch ? batch - b0 : kGemvMaxBatch);
      const uint16_t* xb = x + (uint64_t)b0 * w.k;
      float* yb = y + (uint64_t)b0 * (uint64_t)ldy;
      if (w.layout == 0) {
        GemvGroup grp;
        std::memset(&grp, 0, sizeof(grp));
        grp.w[0] = w;
        grp.col0[0] = col0;
        grp.count = 1;
        uint64_t pipe_blocks = 0;
        int pipe_wpb = 0;
        if (gemv_group_plan(grp, nb, &pipe_blocks, &pipe_wpb)) {
          hipError_t e = launch_gemv_group(grp, w.fmt, xb, nb, yb, ldy, pipe_blocks, pipe_wpb, s);
          if (e != hipSuccess) return e;
        } else {
          GemvNkFn f = w.fmt == kFmtBf16 ? gemv_nk_any_fn<kFmtBf16>(nb)
                       : w.fmt == kFmtExp ? gemv_nk_any_fn<kFmtExp>(nb)
                       : w.fmt == kFmtPal ? gemv_nk_any_fn<kFmtPal>(nb) : gemv_nk_any_fn<kFmtPalRun>(nb);
          uint64_t blocks = (w.n + 3) / 4;
          if (blocks > 8192) blocks = 8192;
          hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(256), 0, s, w, xb, nb, yb, ldy, col0);
        }
      } else {
        const int slices = kn_slices(w, nb, cfg);
        if (partial == nullptr || partial_elems < (size_t)slices * (size_t)nb * w.n) return hipErrorInvalidValue;
        const uint64_t pairs = (w.k + 1) / 2;
        const uint32_t pps = (uint32_t)((pairs + (uint64_t)slices - 1) / (uint64_t)slices);
        const unsigned gy = (unsigned)((pairs + pps - 1) / pps);
        GemvKnFn f = w.fmt == kFmtBf16 ? gemv_kn_fn<kFmtBf16>(nb, w.n)
                     : w.fmt == kFmtExp ? gemv_kn_fn<kFmtExp>(nb, w.n)
                     : w.fmt == kFmtPal ? gemv_kn_fn<kFmtPal>(nb, w.n) : gemv_kn_fn<kFmtPalRun>(nb, w.n);
        const uint64_t bw = 64u * (uint64_t)kn_ow(nb);
        hipLaunchKernelGGL(f, dim3((unsigned)((w.n + bw - 1) / bw), gy), dim3(512), (size_t)nb * pps * 4u, s, w, xb, nb,
                           partial, pps);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_sum_slices(partial, (int)gy, w.n, nb, yb, ldy, col0, s);
        if (e != hipSuccess) return e;
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (!gemm_variant_supported(v, (int)w.layout)) return hipErrorNotSupported;
  if (gemm_variant_is_rf(v))
    return launch_mfma_rf(w, x, batch, y, ldy, col0, v - rf_first_variant(), cfg ? cfg->split_k : 0, device_cus(),
                          partial, partial_elems, s);
  return launch_mfma2(w, x, batch, y, ldy, col0, gemm_variant_tile(v), cfg ? cfg->split_k : 0, partial, partial_elems,
                      s);
}

}  // namespace uw
