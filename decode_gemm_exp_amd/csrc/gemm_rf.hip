// gemm_rf.hip -- register-fed reconstructive MFMA GEMM for small batches
// (up to 64 rows of x per launch), y = x . W^T with W stored [N][K].
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "重建矩陣乘法核心運作": the
// compressed weights are rebuilt to BF16 on chip and fed straight to the
// matrix units; section "四種執行管道" lists the weight forms the matmul
// reads (BF16, exponent + sign/mantissa, palette + sign/mantissa).
//
// At small batch the matmul is a stream over the weights: every weight is used
// by at most 64 rows of x, so the kernel is designed to keep many bytes of
// compressed weights in flight rather than to reuse tiles.
//   * No block-wide LDS staging: each wave loads its weights straight into
//     registers, rebuilds BF16 there and issues v_mfma_f32_16x16x32_bf16 with
//     the rebuilt weights as the A operand (16 output features) and x as the
//     B operand (16 batch rows per MFMA, up to four groups of 16).
//   * The order of k inside an MFMA is free as long as A and B agree, so lane
//     group g (= lane / 16) of a wave takes 32 consecutive k of its row in a
//     128-wide window: the four lane groups read one whole 128-byte line of
//     sign+mantissa bytes per row, and MFMA m of the window takes the lane's
//     weights 8m .. 8m+7.  The lane loads the matching 64 bytes of each x row.
//   * A wave owns R row tiles (16 R output features) and walks the windows
//     wave, wave + 4, ... of its K range, double buffered in registers; the
//     palette format's verbatim flag and rank words are loaded one window
//     ahead of the data, so a verbatim group's exponents are requested from
//     the side section directly.
//   * The four waves of a block cover the same rows and interleaved windows;
//     their partial sums meet in LDS and are added in a fixed order.  K may be
//     split further over grid.y, then a fixed-order reduction adds the slices.
#include <algorithm>

#include "rebuild.h"

namespace uw {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWin = 128;   // k per window (32 per lane group)

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Which 32 weights of a 128-wide window lane group g (= lane / 16) owns:
//   BF16 (two bytes a weight): MFMA m takes k0 + 32 m + 8 g .. +7, so every
//   load instruction reads 64 contiguous bytes of each of its 16 rows;
//   byte formats: lane group g takes k0 + 32 g .. +31, all in one group, and
//   MFMA m its weights 8 m .. +7.  A lane's 32 index nibbles are then one
//   aligned 16-byte load and its group's verbatim flag one bit.
// The x fragment of MFMA m uses the same k (kx_off).
template <int FMT>
__device__ __forceinline__ int kx_off(int m, int g) {
  return FMT == kFmtBf16 ? 32 * m + 8 * g : 32 * g + 8 * m;
}

// Compressed data of one lane's 32 weights of one row.
//   bf16: w[m] = the 8 weights of MFMA m
//   exp:  s0, s1 = the 32 sign+mantissa bytes, e0, e1 = the 32 exponent bytes
//   pal:  s0, s1 as above; e0 = the 16 index bytes (32 nibbles), e1 = zero;
//         or, when the lane's group is verbatim, e0, e1 = its 32 exponent bytes
struct Raw32 {
  uint4 s0, s1, e0, e1;
};

// An offset past the end of every buffer resource: its loads return zero
// without touching memory.
constexpr uint32_t kRfPastEnd = 0x7FFF0000u;
constexpr uint64_t kRfVexpMax = 0x40000000u;   // the verbatim section's resource spans at most 1 GiB
typedef unsigned int u32x4_rf __attribute__((ext_vector_type(4)));

// Loads of one lane's 32 weights of a row; el = stored index of the window
// start plus 32 g (byte formats) or 8 g (BF16).  ok0 / ok1: the window's first
// / second 64 weights exist (byte formats: the lane's group is the window's
// first for lane groups 0 and 1, its second for 2 and 3).  Invalid pieces read
// index 0 (valid memory) and are zeroed when rebuilt.  fw / fh are the
// verbatim flag words holding the window's first and second group (the same
// word unless the pair straddles two), rw the rank word of the first; rvx
// covers the verbatim section.
// The palette formats issue three loads per 32 weights: the second half of a
// verbatim group's exponents comes through rvx at an offset past its end for
// every other lane, so no memory is read for it.  Loading it for every lane,
// or the quarter pieces of both groups that lane pairs used to read twice,
// took a fourth load instruction: 70B gate, palette-direct, x shared through
// LDS, 8 / 32 / 64 rows 85 / 96.7 / 114.5 -> 79.8 / 91.4 / 110.7 us.
template <int FMT>
__device__ __forceinline__ void load32(const WeightView& w, uint64_t el, bool ok0, bool ok1, uint32_t fw, uint32_t fh,
                                       uint32_t rw, int g, __amdgpu_buffer_rsrc_t rvx, Raw32& r, uint32_t& verb) {
  verb = 0;
  if constexpr (FMT == kFmtBf16) {
    const uint64_t a = ok0 ? el : 0, b = ok1 ? el + 64 : 0;
    r.s0 = *reinterpret_cast<const uint4*>(w.bf16 + a);
    r.s1 = *reinterpret_cast<const uint4*>(w.bf16 + a + 32);
    r.e0 = *reinterpret_cast<const uint4*>(w.bf16 + b);
    r.e1 = *reinterpret_cast<const uint4*>(w.bf16 + b + 32);
  } else {
    const bool second = g >= 2;   // the lane's weights lie in the window's second group
    const bool ok = second ? ok1 : ok0;
    const uint64_t a = ok ? el : 0;
    r.s0 = *reinterpret_cast<const uint4*>(w.sm + a);
    r.s1 = *reinterpret_cast<const uint4*>(w.sm + a + 16);
    if constexpr (FMT == kFmtExp) {
      r.e0 = *reinterpret_cast<const uint4*>(w.ex + a);
      r.e1 = *reinterpret_cast<const uint4*>(w.ex + a + 16);
    } else {
      const uint64_t gl = el >> 6;                 // the lane's group
      const uint64_t g0 = second ? gl - 1 : gl;    // the window's first group
      const bool v = ok & group_verbatim(second ? fh : fw, gl);
      const uint32_t rk = group_rank(fw, rw, g0) + (second && group_verbatim(fw, g0) ? 1u : 0u);
      const uint32_t vo = rk * 64u + (uint32_t)(el & 63);   // the lane's exponents in the verbatim section
      // a is a multiple of 32 weights, so the 16 index bytes are aligned
      r.e0 = *reinterpret_cast<const uint4*>(v ? w.vexp + vo : w.pidx + (a >> 1));
      const u32x4_rf q = __builtin_amdgcn_raw_buffer_load_b128(rvx, (int)(v ? vo + 16u : kRfPastEnd), 0, 0);
      r.e1 = make_uint4(q.x, q.y, q.z, q.w);
      verb = v ? 1u : 0u;
    }
  }
}

// A operand of MFMA m as BF16 (ok: the weights it takes exist)
template <int FMT>
__device__ __forceinline__ bf16x8 a_frag(const WeightView& w, const Raw32& r, uint32_t verb, bool ok, int m) {
  uint4 o;
  if constexpr (FMT == kFmtBf16) {
    o = m == 0 ? r.s0 : m == 1 ? r.s1 : m == 2 ? r.e0 : r.e1;
  } else {
    // weights 8 m .. +7 of the lane's 32: words 2 (m % 2) and 2 (m % 2) + 1
    // of the 16-byte half m / 2
    const uint4& sp = (m >> 1) ? r.s1 : r.s0;
    const int wi = 2 * (m & 1);
    const uint32_t s0 = word(sp, wi), s1 = word(sp, wi + 1);
    uint32_t e0, e1;
    if constexpr (FMT == kFmtExp) {
      const uint4& ep = (m >> 1) ? r.e1 : r.e0;
      e0 = word(ep, wi);
      e1 = word(ep, wi + 1);
    } else {
      pal8<FMT == kFmtPalRun>(word(r.e0, m), w.pal, e0, e1);
      const uint4& ep = (m >> 1) ? r.e1 : r.e0;   // verbatim: the exponent bytes
      e0 = verb ? word(ep, wi) : e0;
      e1 = verb ? word(ep, wi + 1) : e1;
    }
    rebuild4(s0, e0, o.x, o.y);
    rebuild4(s1, e1, o.z, o.w);
  }
  o.x = ok ? o.x : 0u;
  o.y = ok ? o.y : 0u;
  o.z = ok ? o.z : 0u;
  o.w = ok ? o.w : 0u;
  return __builtin_bit_cast(bf16x8, o);
}

template <int FMT, int R, int NBG, bool XS = (NBG >= 2)>
__global__ __launch_bounds__(256) void k_mfma_rf(WeightView w, const uint16_t* __restrict__ x, int B,
                                                 float* __restrict__ y, int64_t ldy, int64_t col0, int64_t kslice,
                                                 float* __restrict__ part, uint32_t fwords,
                                                 const uint4* __restrict__ xp) {
  constexpr int SLOT = R * NBG * 64;   // float4 per wave in the reduction buffer
  __shared__ f32x4 red[4 * SLOT];
  extern __shared__ uint32_t fl[];     // palette: the block's verbatim flag words, then their rank words
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t rvx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w.vexp), (short)0, (int)(fmt_is_pal(FMT) ? w.vexp_bytes : 0u), 0x00020000);
  const int64_t N = (int64_t)w.n, K = (int64_t)w.k;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * R);
  const int64_t kb = (int64_t)blockIdx.y * kslice;
  const int64_t ke = kb + kslice < K ? kb + kslice : K;
  const int nwin = (int)((ke - kb + kWin - 1) / kWin);
  const int mine = nwin > wave ? (nwin - wave + 3) / 4 : 0;   // windows wave, wave + 4, ...

  // The block's rows are contiguous in storage, so the flag and rank words of
  // their groups are too: at most fwords of each, staged in LDS once.
  uint64_t fbase = 0;
  if constexpr (fmt_is_pal(FMT)) {
    const int64_t nl = n0 + 16 * R < N ? n0 + 16 * R : N;
    fbase = (uint64_t)(n0 * K) >> 11;
    const uint32_t cnt = (uint32_t)((((uint64_t)(nl * K) + 2047) >> 11) - fbase);
    for (uint32_t i = threadIdx.x; i < cnt; i += 256) {
      fl[i] = w.vflags[fbase + i];
      fl[fwords + i] = w.vrank[fbase + i];
    }
    __syncthreads();
  }

  // x rows of this lane (rows past the batch are clamped: their columns are never stored)
  int64_t xrow[NBG];
#pragma unroll
  for (int q = 0; q < NBG; ++q) {
    const int b = 16 * q + i16;
    xrow[q] = (int64_t)(b < B ? b : B - 1) * K;
  }

  // each block starts its walk at a different window, so the chip's
  // concurrent reads spread over the memory channels instead of all rows
  // being read at the same column offset
  const int rot = mine > 0 ? (int)((blockIdx.x * 5u + blockIdx.y * 3u) % (unsigned)mine) : 0;
  auto win_k = [&](int j) __attribute__((always_inline)) {
    int jj = j + rot;
    jj -= jj >= mine ? mine : 0;
    return kb + (int64_t)kWin * (wave + 4 * jj);
  };
  const int goff = FMT == kFmtBf16 ? 8 * g : 32 * g;   // lane group's offset in a window
  // flag and rank words of a window's groups (from LDS).  With K / 64 odd,
  // the two groups of a window may straddle two flag words.
  auto load_flags = [&](int j, uint32_t (&fw)[R], uint32_t (&fh)[R], uint32_t (&rw)[R]) __attribute__((always_inline)) {
    if constexpr (fmt_is_pal(FMT)) {
      const int64_t k0 = win_k(j);
      const bool kv = (j < mine) & (k0 < ke);
      const bool h1 = k0 + 64 < ke;
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int64_t n = n0 + 16 * t + i16;
        const bool v = kv & (n < N);
        const uint64_t g0 = (uint64_t)(n * K + k0) >> 6;
        const uint32_t fi = v ? (uint32_t)((g0 >> 5) - fbase) : 0u;
        const uint32_t fj = (v & h1 & ((g0 & 31) == 31)) ? fi + 1 : fi;
        fw[t] = fl[fi];
        fh[t] = fl[fj];
        rw[t] = fl[fwords + fi];
      }
    }
  };
  // x fragments of window j (the window's MFMA operands, from the packed copy when there is one)
  auto load_x = [&](int j, uint4 (&xr)[NBG][4]) __attribute__((always_inline)) {
    const int64_t k0 = win_k(j);
    const bool kv = (j < mine) & (k0 < ke);
    const bool h1 = k0 + 64 < ke;
    const int64_t kx = kv ? k0 : 0;
    const uint64_t wabs = (uint64_t)(kx / kWin);   // window index along K (packed x)
#pragma unroll
    for (int q = 0; q < NBG; ++q)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t kk = (kv & (h1 | (kx_off<FMT>(m, g) < 64))) ? kx + kx_off<FMT>(m, g) : 0;
        const uint4* pa = xp ? xp + ((wabs * NBG + q) * 4 + m) * 64 + lane
                             : reinterpret_cast<const uint4*>(x + xrow[q] + kk);
        const uint4 v = *pa;
        xr[q][m] = v;
      }
  };
  // okbits: bit 2t = row tile t's first 64 weights exist, bit 2t+1 = its second 64
  auto load_win = [&](int j, Raw32 (&r)[R], uint4 (&xr)[NBG][4], const uint32_t (&fw)[R], const uint32_t (&fh)[R],
                      const uint32_t (&rw)[R], uint32_t& vbits, uint32_t& okbits) __attribute__((always_inline)) {
    const int64_t k0 = win_k(j);
    const bool kv = (j < mine) & (k0 < ke);
    const bool h1 = k0 + 64 < ke;
    vbits = 0;
    okbits = 0;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int64_t n = n0 + 16 * t + i16;
      const bool v = kv & (n < N);
      uint32_t vb;
      load32<FMT>(w, (uint64_t)(n * K + k0 + goff), v, v & h1, fmt_is_pal(FMT) ? fw[t] : 0u,
                  fmt_is_pal(FMT) ? fh[t] : 0u, fmt_is_pal(FMT) ? rw[t] : 0u, g, rvx, r[t], vb);
      vbits |= vb << (2 * t);
      okbits |= (v ? 1u : 0u) << (2 * t);
      okbits |= (v & h1 ? 1u : 0u) << (2 * t + 1);
    }
    if constexpr (!XS) load_x(j, xr);
  };

  f32x4 acc[R][NBG];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int q = 0; q < NBG; ++q) acc[t][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto xbuf_b = [](uint4 (&a)[NBG][4], auto& b) __attribute__((always_inline)) -> uint4 (&)[NBG][4] {
    if constexpr (XS) return a;
    else return b;
  };
  auto compute = [&](const Raw32 (&r)[R], const uint4 (&xr)[NBG][4], uint32_t vbits,
                     uint32_t okbits) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < R; ++t) {
        // the piece holding MFMA m: BF16 first half m < 2, byte formats piece m / 2
        // the weights exist: BF16, the window half of MFMA m; byte formats,
        // the half holding the lane's group
        const bool ok = (okbits >> (2 * t + (FMT == kFmtBf16 ? (m >> 1) : (g >> 1)))) & 1u;
        const bf16x8 a = a_frag<FMT>(w, r[t], (vbits >> (2 * t)) & 1u, ok, m);
#pragma unroll
        for (int q = 0; q < NBG; ++q)
          acc[t][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, xr[q][m]), acc[t][q],
                                                              0, 0, 0);
      }
  };

  // two windows in registers: the loads of window j+2 (and the flag words of
  // j+4) are issued as soon as window j has been consumed.  Windows past the
  // range load index 0 and add zeros, so the loop has no tail.
  // With XS (two or more batch groups) x is single buffered, one window
  // ahead: it comes from L2, and a second buffer would cost the registers
  // that keep two windows of weights in flight.
  Raw32 rA[R], rB[R];
  uint4 xA[NBG][4], xB[XS ? 1 : NBG][4];
  uint32_t fA[R], hA[R], gA[R], fB[R], hB[R], gB[R];
  uint32_t vA, oA, vB, oB;
#pragma unroll
  for (int t = 0; t < R; ++t) fA[t] = hA[t] = gA[t] = fB[t] = hB[t] = gB[t] = 0u;
  // the prologue issues its loads in the loop's order (A before B), so the
  // waits at the loop head can count only the loads it needs
  load_flags(0, fA, hA, gA);
  load_flags(1, fB, hB, gB);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XS) load_x(0, xA);
  load_win(0, rA, xA, fA, hA, gA, vA, oA);
  load_flags(2, fA, hA, gA);
  __builtin_amdgcn_sched_barrier(0);
  load_win(1, rB, xbuf_b(xA, xB), fB, hB, gB, vB, oB);
  load_flags(3, fB, hB, gB);
  __builtin_amdgcn_sched_barrier(0);
  // (the scheduling barriers keep each buffer's reloads behind the MFMAs that
  // read it: hoisted above them, the loads land in other registers and the
  // loop's back edge has to wait for every load in flight)
  // (a do-while: with no guard in front of the loop, the compiler cannot sink
  // the prologue's x loads behind the second window's weights)
  int j = 0;
  do {
    compute(rA, xA, vA, oA);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XS) load_x(j + 1, xA);
    load_win(j + 2, rA, xA, fA, hA, gA, vA, oA);
    load_flags(j + 4, fA, hA, gA);
    __builtin_amdgcn_sched_barrier(0);
    compute(rB, xbuf_b(xA, xB), vB, oB);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XS) load_x(j + 2, xA);
    load_win(j + 3, rB, xbuf_b(xA, xB), fB, hB, gB, vB, oB);
    load_flags(j + 5, fB, hB, gB);
    __builtin_amdgcn_sched_barrier(0);
    j += 2;
  } while (j < mine);

  // the four waves' sums, added in wave order.  D of v_mfma_f32_16x16x32_bf16:
  // lane l holds rows 4 (l / 16) .. +3 (output features) of column l % 16 (batch row)
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int q = 0; q < NBG; ++q) red[wave * SLOT + (t * NBG + q) * 64 + lane] = acc[t][q];
  __syncthreads();
  float* out = part ? part + (uint64_t)blockIdx.y * (uint64_t)B * (uint64_t)N : y + col0;
  const int64_t ld = part ? N : ldy;
  for (int e = threadIdx.x; e < SLOT; e += 256) {
    const f32x4 s = ((red[e] + red[SLOT + e]) + red[2 * SLOT + e]) + red[3 * SLOT + e];
    const int ln = e & 63, tq = e >> 6, q = tq % NBG, t = tq / NBG;
    const int64_t n = n0 + 16 * t + 4 * (ln >> 4);
    const int b = 16 * q + (ln & 15);
    if (b < B) {
      float* o = out + (int64_t)b * ld + n;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) o[r] = s[r];
    }
  }
}

// x in the order the kernel's lanes read it: entry ((w * NBG + q) * 4 + m) * 64
// + lane holds the 8 x values of batch row 16 q + lane % 16 (clamped to the
// last row) that MFMA m of window w multiplies, so each of the kernel's x
// loads reads 1 KB of contiguous memory instead of 16 rows in 16-byte pieces.
template <int FMT>
__global__ __launch_bounds__(256) void k_rf_pack_x(const uint16_t* __restrict__ x, int B, int64_t K, int nbg,
                                                   uint4* __restrict__ xp, uint64_t entries) {
  for (uint64_t e = (uint64_t)blockIdx.x * 256 + threadIdx.x; e < entries; e += (uint64_t)gridDim.x * 256) {
    const int lane = (int)(e & 63), m = (int)((e >> 6) & 3);
    const uint64_t r = e >> 8;
    const int q = (int)(r % (uint64_t)nbg);
    const int64_t wabs = (int64_t)(r / (uint64_t)nbg);
    const int b0 = 16 * q + (lane & 15), b = b0 < B ? b0 : B - 1;
    const int64_t k = wabs * kWin + kx_off<FMT>(m, lane >> 4);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k + 8 <= K) v = *reinterpret_cast<const uint4*>(x + (int64_t)b * K + k);
    xp[e] = v;
  }
}

// Register-fed kernel with x shared through LDS (kinds 2 and 3).  The four
// waves of a block own different rows (wave w: R row tiles from
// 16 R w) and walk the same windows of the block's K range together, so each
// window's x fragments are read from memory once per block, a quarter by
// each wave, into a double-buffered LDS stage, and every wave reads them
// from there.  In the kernel above every wave loads its own windows' x from
// L2: at 64 rows that is 16 KB per window per wave, more than the wave's
// compressed weights, and with x loads taken out (a timing copy) it ran
// 133 -> 84 us on the 70B gate, palette-direct.  One barrier per window: a
// window's x is stored in the half step after it is read from memory and
// read in the next, and a buffer is rewritten only after the barrier that
// follows its last reads.  No cross-wave reduction: each wave stores its
// own rows.  x comes packed (k_rf_pack_x), one window contiguous.
template <int FMT, int R, int NBG, int DP>
__global__ __launch_bounds__(256) void k_mfma_rfx(WeightView w, int B, float* __restrict__ y, int64_t ldy,
                                                  int64_t col0, int64_t kslice, float* __restrict__ part,
                                                  uint32_t fwords, const uint4* __restrict__ xp) {
  static_assert(DP % 2 == 0, "x buffers alternate with the windows");
  constexpr int XE = NBG * 4 * 64;   // uint4 entries of x per window
  extern __shared__ u32x4 dyn4[];
  u32x4* const xs = dyn4;                                          // two windows of x fragments
  uint32_t* const fl = reinterpret_cast<uint32_t*>(dyn4 + 2 * XE);   // palette: flag words, then rank words
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const __amdgpu_buffer_rsrc_t rvx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(w.vexp), (short)0, (int)(fmt_is_pal(FMT) ? w.vexp_bytes : 0u), 0x00020000);
  const int64_t N = (int64_t)w.n, K = (int64_t)w.k;
  const int64_t nblk = (int64_t)blockIdx.x * (64 * R);   // the block's first row
  const int64_t n0 = nblk + (int64_t)wave * (16 * R);    // the wave's first row
  const int64_t kb = (int64_t)blockIdx.y * kslice;
  const int64_t ke = kb + kslice < K ? kb + kslice : K;
  const int nwin = (int)((ke - kb + kWin - 1) / kWin);

  uint64_t fbase = 0;
  if constexpr (fmt_is_pal(FMT)) {
    const int64_t nl = nblk + 64 * R < N ? nblk + 64 * R : N;
    fbase = (uint64_t)(nblk * K) >> 11;
    const uint32_t cnt = (uint32_t)((((uint64_t)(nl * K) + 2047) >> 11) - fbase);
    for (uint32_t i = threadIdx.x; i < cnt; i += 256) {
      fl[i] = w.vflags[fbase + i];
      fl[fwords + i] = w.vrank[fbase + i];
    }
    __syncthreads();
  }

  // blocks start their walks at different windows (reads spread over channels)
  const int rot = nwin > 0 ? (int)((blockIdx.x * 5u + blockIdx.y * 3u) % (unsigned)nwin) : 0;
  auto win_k = [&](int j) __attribute__((always_inline)) {
    int jj = j + rot;
    jj -= jj >= nwin ? nwin : 0;
    return kb + (int64_t)kWin * jj;
  };
  const int goff = FMT == kFmtBf16 ? 8 * g : 32 * g;
  auto load_flags = [&](int j, uint32_t (&fw)[R], uint32_t (&fh)[R], uint32_t (&rw)[R]) __attribute__((always_inline)) {
    if constexpr (fmt_is_pal(FMT)) {
      const int64_t k0 = win_k(j);
      const bool kv = (j < nwin) & (k0 < ke);
      const bool h1 = k0 + 64 < ke;
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int64_t n = n0 + 16 * t + i16;
        const bool v = kv & (n < N);
        const uint64_t g0 = (uint64_t)(n * K + k0) >> 6;
        const uint32_t fi = v ? (uint32_t)((g0 >> 5) - fbase) : 0u;
        const uint32_t fj = (v & h1 & ((g0 & 31) == 31)) ? fi + 1 : fi;
        fw[t] = fl[fi];
        fh[t] = fl[fj];
        rw[t] = fl[fwords + fi];
      }
    }
  };
  auto load_win = [&](int j, Raw32 (&r)[R], const uint32_t (&fw)[R], const uint32_t (&fh)[R],
                      const uint32_t (&rw)[R], uint32_t& vbits, uint32_t& okbits) __attribute__((always_inline)) {
    const int64_t k0 = win_k(j);
    const bool kv = (j < nwin) & (k0 < ke);
    const bool h1 = k0 + 64 < ke;
    vbits = 0;
    okbits = 0;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int64_t n = n0 + 16 * t + i16;
      const bool v = kv & (n < N);
      uint32_t vb;
      load32<FMT>(w, (uint64_t)(n * K + k0 + goff), v, v & h1, fmt_is_pal(FMT) ? fw[t] : 0u,
                  fmt_is_pal(FMT) ? fh[t] : 0u, fmt_is_pal(FMT) ? rw[t] : 0u, g, rvx, r[t], vb);
      vbits |= vb << (2 * t);
      okbits |= (v ? 1u : 0u) << (2 * t);
      okbits |= (v & h1 ? 1u : 0u) << (2 * t + 1);
    }
  };
  // this thread's share of a window's packed x (windows past the range read
  // window 0: their weights are zero)
  auto load_xs = [&](int j, u32x4 (&xg)[NBG]) __attribute__((always_inline)) {
    const int64_t k0 = win_k(j);
    const bool kv = (j < nwin) & (k0 < ke);
    const u32x4* src = reinterpret_cast<const u32x4*>(xp) + (uint64_t)(kv ? k0 / kWin : 0) * XE + threadIdx.x;
#pragma unroll
    for (int i = 0; i < NBG; ++i) xg[i] = src[256 * i];
  };
  auto store_xs = [&](int buf, const u32x4 (&xg)[NBG]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NBG; ++i) xs[buf * XE + 256 * i + (int)threadIdx.x] = xg[i];
  };

  f32x4 acc[R][NBG];
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int q = 0; q < NBG; ++q) acc[t][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Raw32 (&r)[R], int buf, uint32_t vbits, uint32_t okbits) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x4 xr[NBG];
#pragma unroll
      for (int q = 0; q < NBG; ++q) xr[q] = xs[buf * XE + (q * 4 + m) * 64 + lane];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        // the weights exist: BF16, the window half of MFMA m; byte formats,
        // the half holding the lane's group
        const bool ok = (okbits >> (2 * t + (FMT == kFmtBf16 ? (m >> 1) : (g >> 1)))) & 1u;
        const bf16x8 a = a_frag<FMT>(w, r[t], (vbits >> (2 * t)) & 1u, ok, m);
#pragma unroll
        for (int q = 0; q < NBG; ++q)
          acc[t][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, xr[q]), acc[t][q], 0, 0, 0);
      }
    }
  };

  // DP windows of weights in registers: the loads of window j + DP (and the
  // flag words of j + 2 DP) are issued as soon as window j has been consumed;
  // x is staged one window ahead.  Windows past the range load index 0 and
  // add zeros, so the loop has no tail.
  Raw32 rw[DP][R];
  u32x4 xg[NBG];
  uint32_t fw[DP][R], fh[DP][R], fr[DP][R];
  uint32_t vb[DP], ob[DP];
#pragma unroll
  for (int d = 0; d < DP; ++d)
#pragma unroll
    for (int t = 0; t < R; ++t) fw[d][t] = fh[d][t] = fr[d][t] = 0u;
#pragma unroll
  for (int d = 0; d < DP; ++d) load_flags(d, fw[d], fh[d], fr[d]);
  __builtin_amdgcn_sched_barrier(0);
  load_xs(0, xg);
#pragma unroll
  for (int d = 0; d < DP; ++d) {
    load_win(d, rw[d], fw[d], fh[d], fr[d], vb[d], ob[d]);
    load_flags(d + DP, fw[d], fh[d], fr[d]);
  }
  __builtin_amdgcn_sched_barrier(0);
  store_xs(0, xg);
  load_xs(1, xg);
  __syncthreads();
  int j = 0;
  do {
#pragma unroll
    for (int d = 0; d < DP; ++d) {   // window j + d, its x in buffer d % 2 (DP is even)
      compute(rw[d], d & 1, vb[d], ob[d]);
      __builtin_amdgcn_sched_barrier(0);
      load_win(j + d + DP, rw[d], fw[d], fh[d], fr[d], vb[d], ob[d]);
      load_flags(j + d + 2 * DP, fw[d], fh[d], fr[d]);
      __builtin_amdgcn_sched_barrier(0);
      store_xs((d + 1) & 1, xg);   // window j + d + 1
      load_xs(j + d + 2, xg);
      __syncthreads();
    }
    j += DP;
  } while (j < nwin);

  // D of v_mfma_f32_16x16x32_bf16: lane l holds rows 4 (l / 16) .. +3 (output
  // features) of column l % 16 (batch row)
  float* out = part ? part + (uint64_t)blockIdx.y * (uint64_t)B * (uint64_t)N : y + col0;
  const int64_t ld = part ? N : ldy;
#pragma unroll
  for (int t = 0; t < R; ++t)
#pragma unroll
    for (int q = 0; q < NBG; ++q) {
      const int64_t n = n0 + 16 * t + 4 * (lane >> 4);
      const int b = 16 * q + i16;
      if (b < B) {
        float* o = out + (int64_t)b * ld + n;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) o[r] = acc[t][q][r];
      }
    }
}

typedef void (*RfxFn)(WeightView, int, float*, int64_t, int64_t, int64_t, float*, uint32_t, const uint4*);

constexpr int kRfxDepth = 2;   // windows of weights in flight per wave

template <int F, int R>
RfxFn rfx_fn(int nbg) {
  if (nbg <= 1) return k_mfma_rfx<F, R, 1, kRfxDepth>;
  if (nbg <= 2) return k_mfma_rfx<F, R, 2, kRfxDepth>;
  return k_mfma_rfx<F, R, 4, kRfxDepth>;
}

template <int R>
RfxFn rfx_pick(int fmt, int nbg) {
  return fmt == kFmtBf16 ? rfx_fn<kFmtBf16, R>(nbg)
         : fmt == kFmtExp ? rfx_fn<kFmtExp, R>(nbg)
         : fmt == kFmtPal ? rfx_fn<kFmtPal, R>(nbg) : rfx_fn<kFmtPalRun, R>(nbg);
}

typedef void (*RfFn)(WeightView, const uint16_t*, int, float*, int64_t, int64_t, int64_t, float*, uint32_t,
                     const uint4*);

template <int F, int R>
RfFn rf_fn(int nbg) {
  if (nbg <= 1) return k_mfma_rf<F, R, 1>;
  if (nbg <= 2) return k_mfma_rf<F, R, 2>;
  return k_mfma_rf<F, R, 4>;
}

template <int R>
RfFn rf_pick(int fmt, int nbg) {
  return fmt == kFmtBf16 ? rf_fn<kFmtBf16, R>(nbg)
         : fmt == kFmtExp ? rf_fn<kFmtExp, R>(nbg)
         : fmt == kFmtPal ? rf_fn<kFmtPal, R>(nbg) : rf_fn<kFmtPalRun, R>(nbg);
}

constexpr int kRfMaxBatch = 64;
constexpr uint64_t kRfMaxFlagLds = 64 * 1024;   // bytes of staged flag and rank words (K up to 256 Ki at 4 row tiles)

int rf_nbg(int64_t nb) { return nb <= 16 ? 1 : nb <= 32 ? 2 : 4; }

}  // namespace

// kinds: 0 and 1, x per wave from L2 with two and four row tiles per wave
// (a block: 32 or 64 rows); 2 and 3, x shared through LDS with one and two
// row tiles per wave (a block: 64 or 128 rows)
int mfma_rf_kinds() { return 4; }
int mfma_rf_max_batch() { return kRfMaxBatch; }
static bool rf_shared_x(int kind) { return kind >= 2; }
static int rf_tiles(int kind) { return kind == 0 ? 2 : kind == 1 ? 4 : kind == 2 ? 1 : 2; }   // per wave
static int64_t rf_block_rows(int kind) { return 16 * (int64_t)rf_tiles(kind) * (rf_shared_x(kind) ? 4 : 1); }

// K slices over grid.y: none unless the row blocks leave the chip under two
// blocks per CU (one for the shared-x kinds), and never below 16 windows per
// slice (4 per wave when the waves take turns, 16 when they walk the windows
// together).  The shared-x kinds gain less from a second block per CU than
// the partial sums cost: 70B gate (448 64-row blocks), palette-direct, 16
// rows: 81 us unsplit, 92 us in two slices.
int mfma_rf_slices(const WeightView& w, int kind, int split_hint, int cus) {
  const int64_t rowblocks = ((int64_t)w.n + rf_block_rows(kind) - 1) / rf_block_rows(kind);
  const int64_t wins = ((int64_t)w.k + kWin - 1) / kWin;
  const int64_t cover = rf_shared_x(kind) ? cus : 2 * (int64_t)cus;
  int s = 1;
  if (split_hint > 0) {
    s = split_hint;
  } else {
    while (rowblocks * s < cover && wins / (2 * s) >= 16) s *= 2;
  }
  if (s > wins) s = (int)wins;
  if (s < 1) s = 1;
  return s;
}

// x is packed (k_rf_pack_x) for launches of more than 8 rows, and always for
// the shared-x kinds: below that the rows past the batch repeat the last one
// and the plain loads are cheaper
static bool rf_packs(int kind, int64_t nb) { return rf_shared_x(kind) || nb > 8; }
static size_t rf_part_floats(const WeightView& w, int slices, int64_t nb) {   // 16-byte multiple
  return slices > 1 ? ((size_t)slices * (size_t)nb * (size_t)w.n + 3) & ~(size_t)3 : 0;
}
static size_t rf_pack_entries(const WeightView& w, int kind, int64_t nb) {
  const int64_t wins = ((int64_t)w.k + kWin - 1) / kWin;
  return rf_packs(kind, nb) ? (size_t)wins * (size_t)rf_nbg(nb) * 4 * 64 : 0;
}

size_t mfma_rf_partial_elems(const WeightView& w, int64_t batch, int kind, int split_hint, int cus) {
  const int s = mfma_rf_slices(w, kind, split_hint, cus);
  const int64_t nb = batch < kRfMaxBatch ? batch : kRfMaxBatch;
  return rf_part_floats(w, s, nb) + 4 * rf_pack_entries(w, kind, nb);
}

// flag and rank words one block stages (palette formats)
static uint64_t rf_flag_words(const WeightView& w, int kind) {
  return fmt_is_pal(w.fmt) ? (uint64_t)rf_block_rows(kind) * w.k / 2048 + 2 : 0;
}

bool mfma_rf_supported(const WeightView& w, int kind) {
  return w.layout == 0 && rf_flag_words(w, kind) * 8 <= kRfMaxFlagLds &&
         (!fmt_is_pal(w.fmt) || w.vexp_bytes <= kRfVexpMax);
}

hipError_t launch_mfma_rf(const WeightView& w, const uint16_t* x, int64_t batch, float* y, int64_t ldy,
                          int64_t col0, int kind, int split_hint, int cus, float* part, size_t part_elems,
                          hipStream_t s) {
  if (!mfma_rf_supported(w, kind)) return hipErrorNotSupported;
  const int slices = mfma_rf_slices(w, kind, split_hint, cus);
  const int64_t wins = ((int64_t)w.k + kWin - 1) / kWin;
  const int64_t kslice = ((wins + slices - 1) / slices) * kWin;
  const unsigned rowblocks = (unsigned)(((int64_t)w.n + rf_block_rows(kind) - 1) / rf_block_rows(kind));
  const uint32_t fwords = (uint32_t)rf_flag_words(w, kind);   // staged in LDS per block
  hipError_t e0 = hipSuccess;
  for (int64_t b0 = 0; b0 < batch; b0 += kRfMaxBatch) {
    const int64_t nb = batch - b0 < kRfMaxBatch ? batch - b0 : kRfMaxBatch;
    const bool split = slices > 1;
    const size_t pf = rf_part_floats(w, slices, nb), pe = rf_pack_entries(w, kind, nb);
    if ((split || pe > 0) && (part == nullptr || part_elems < pf + 4 * pe)) return hipErrorInvalidValue;
    const uint16_t* xb = x + (uint64_t)b0 * w.k;
    float* yb = y + (uint64_t)b0 * (uint64_t)ldy;
    uint4* xp = nullptr;
    if (pe > 0) {
      xp = reinterpret_cast<uint4*>(part + pf);
      const unsigned grid = (unsigned)std::min<size_t>((pe + 255) / 256, 4096);
      if (w.fmt == kFmtBf16)
        hipLaunchKernelGGL(k_rf_pack_x<kFmtBf16>, dim3(grid), dim3(256), 0, s, xb, (int)nb, (int64_t)w.k, rf_nbg(nb),
                           xp, (uint64_t)pe);
      else
        hipLaunchKernelGGL(k_rf_pack_x<kFmtExp>, dim3(grid), dim3(256), 0, s, xb, (int)nb, (int64_t)w.k, rf_nbg(nb),
                           xp, (uint64_t)pe);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const bool first = b0 == 0, last = b0 + kRfMaxBatch >= batch;
    if (rf_shared_x(kind)) {
      const RfxFn f = kind == 2 ? rfx_pick<1>(w.fmt, rf_nbg(nb)) : rfx_pick<2>(w.fmt, rf_nbg(nb));
      const size_t lds = 2 * (size_t)rf_nbg(nb) * 4 * 64 * sizeof(uint4) + (size_t)fwords * 8;
      e0 = allow_dynamic_lds((const void*)f, (int)lds);
      if (e0 != hipSuccess) return e0;
      if (first) kernel_event_before(s);
      hipLaunchKernelGGL(f, dim3(rowblocks, (unsigned)slices), dim3(256), lds, s, w, (int)nb, yb, ldy, col0, kslice,
                         split ? part : nullptr, fwords, (const uint4*)xp);
    } else {
      const RfFn f = kind == 0 ? rf_pick<2>(w.fmt, rf_nbg(nb)) : rf_pick<4>(w.fmt, rf_nbg(nb));
      e0 = allow_dynamic_lds((const void*)f, (int)(fwords * 8));
      if (e0 != hipSuccess) return e0;
      if (first) kernel_event_before(s);
      hipLaunchKernelGGL(f, dim3(rowblocks, (unsigned)slices), dim3(256), (size_t)fwords * 8, s, w, xb, (int)nb, yb,
                         ldy, col0, kslice, split ? part : nullptr, fwords, (const uint4*)xp);
    }
    hipError_t e = hipGetLastError();
    if (last) kernel_event_after(s);
    if (e != hipSuccess) return e;
    if (split) {
      e = launch_sum_slices(part, slices, w.n, nb, yb, ldy, col0, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace uw
