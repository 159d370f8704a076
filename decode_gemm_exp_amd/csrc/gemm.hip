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
//   * GEMV (batch <= 8): VALU, v_dot2_f32_bf16 on rebuilt pairs.  NK: one
//     wave per output row, lanes stride K in 16-weight chunks, wave reduce.
//     KN: lanes own 8 consecutive outputs, waves stride K, partial sums per
//     K slice go to the workspace and a second kernel adds them in a fixed
//     order (deterministic).
//   * MFMA (batch > 8): gemm_mfma.hip.
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

// ---- GEMV, stored [N][K] ----------------------------------------------------------
template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_gemv_nk(WeightView w, const uint16_t* __restrict__ x, int B,
                                                 float* __restrict__ y, int64_t ldy, int64_t col0) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave_id = ((uint64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const uint64_t nwaves = (uint64_t)gridDim.x * 4;
  const uint64_t K = w.k;
  for (uint64_t n = wave_id; n < w.n; n += nwaves) {
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    for (uint64_t k = (uint64_t)lane * 16; k < K; k += 1024) {
      uint32_t wv[8];
      load16<FMT>(w, n * K + k, wv);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < B) {
          const uint4* xp = reinterpret_cast<const uint4*>(x + (uint64_t)b * K + k);
          const uint4 x0 = xp[0], x1 = xp[1];
          float a = acc[b];
          a = dot2(wv[0], x0.x, a); a = dot2(wv[1], x0.y, a);
          a = dot2(wv[2], x0.z, a); a = dot2(wv[3], x0.w, a);
          a = dot2(wv[4], x1.x, a); a = dot2(wv[5], x1.y, a);
          a = dot2(wv[6], x1.z, a); a = dot2(wv[7], x1.w, a);
          acc[b] = a;
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
// grid.x: blocks of 512 outputs (64 lanes x 8); grid.y: K slices.  The 4 waves
// of a block split the slice; their sums meet in LDS; one partial row per
// slice is written to part[slice][b][n].
template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_gemv_kn(WeightView w, const uint16_t* __restrict__ x, int B,
                                                 float* __restrict__ part, int64_t rows_per_slice) {
  __shared__ float red[4][NB][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t N = w.n, K = w.k;
  const uint64_t n0 = (uint64_t)blockIdx.x * 512 + (uint64_t)lane * 8;
  const uint64_t kb = (uint64_t)blockIdx.y * (uint64_t)rows_per_slice;
  const uint64_t ke = min(kb + (uint64_t)rows_per_slice, K);
  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[b][i] = 0.f;
  if (n0 < N) {
    for (uint64_t k = kb + (uint64_t)wave; k < ke; k += 4) {
      uint32_t wv[4];
      load8<FMT>(w, k * N + n0, wv);
      float wf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wf[2 * i] = __uint_as_float(wv[i] << 16);
        wf[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < B) {
          const float xb = __uint_as_float((uint32_t)x[(uint64_t)b * K + k] << 16);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[b][i] = fmaf(xb, wf[i], acc[b][i]);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][b][lane * 8 + i] = acc[b][i];
  __syncthreads();
  for (int t = threadIdx.x; t < NB * 512; t += 256) {
    const int b = t / 512, c = t % 512;
    const uint64_t n = (uint64_t)blockIdx.x * 512 + (uint64_t)c;
    if (b < B && n < N) {
      const float s = ((red[0][b][c] + red[1][b][c]) + red[2][b][c]) + red[3][b][c];
      part[((uint64_t)blockIdx.y * (uint64_t)B + (uint64_t)b) * N + n] = s;
    }
  }
}

__global__ __launch_bounds__(256) void k_reduce_slices(const float* __restrict__ part, int slices, int B,
                                                       uint64_t N, float* __restrict__ y, int64_t ldy,
                                                       int64_t col0) {
  const uint64_t total = (uint64_t)B * N;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (uint64_t)gridDim.x * 256) {
    const uint64_t b = i / N, n = i % N;
    float s = 0.f;
    for (int p = 0; p < slices; ++p) s += part[(uint64_t)p * total + i];
    y[b * (uint64_t)ldy + (uint64_t)col0 + n] = s;
  }
}

typedef void (*GemvNkFn)(WeightView, const uint16_t*, int, float*, int64_t, int64_t);
typedef void (*GemvKnFn)(WeightView, const uint16_t*, int, float*, int64_t);

template <int F>
GemvNkFn gemv_nk_fn(int nb) {
  if (nb <= 1) return k_gemv_nk<F, 1>;
  if (nb <= 2) return k_gemv_nk<F, 2>;
  if (nb <= 4) return k_gemv_nk<F, 4>;
  return k_gemv_nk<F, 8>;
}
template <int F>
GemvKnFn gemv_kn_fn(int nb) {
  if (nb <= 1) return k_gemv_kn<F, 1>;
  if (nb <= 2) return k_gemv_kn<F, 2>;
  if (nb <= 4) return k_gemv_kn<F, 4>;
  return k_gemv_kn<F, 8>;
}

constexpr int kGemvMaxBatch = 8;

// largest MFMA tile whose grid alone covers the chip; else 128 x 128 with split K
int default_tile(uint64_t n, int64_t batch) {
  for (int t = mfma2_tile_count() - 1; t >= 0; --t) {
    const int bm = t == 0 ? 64 : (t == 1 || t == 2) ? 128 : 256;
    const int bn = (t == 2 || t == 4) ? 256 : 128;
    if (bm > 2 * batch && t > 0) continue;   // no tile much taller than the batch
    const uint64_t blocks = (n + bn - 1) / bn * (uint64_t)((batch + bm - 1) / bm);
    if (blocks >= 256) return t;
  }
  return batch <= 64 ? 0 : 1;
}

// K slices of the KN GEMV: enough blocks to cover the chip a few times.
int kn_slices(const WeightView& w, const uw_kernel_cfg* cfg) {
  if (cfg && cfg->split_k > 0) return cfg->split_k;
  const uint64_t nblocks = (w.n + 511) / 512;
  uint64_t s = (1024 + nblocks - 1) / nblocks;
  const uint64_t max_s = (w.k + 63) / 64;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  return (int)s;
}

}  // namespace

// Variant numbering seen through uw_kernel_cfg.variant: 1 = VALU GEMV (any
// batch, eight rows per launch), 2.. = the MFMA tiles of gemm_mfma.hip.
int gemm_variant_count() { return 1 + mfma2_tile_count(); }

static int resolve_variant(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg) {
  if (cfg && cfg->variant > 0 && cfg->variant <= gemm_variant_count()) return cfg->variant;
  return batch <= kGemvMaxBatch ? 1 : 2 + default_tile(w.n, batch);
}

// Workspace floats for partial sums: enough for every variant (the KN GEMV's
// K slices, the MFMA split-K slices), so one size serves any kernel choice.
size_t gemm_partial_elems(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg) {
  size_t need = 0;
  if (w.layout == 1) {
    const int64_t rows = batch < kGemvMaxBatch ? batch : kGemvMaxBatch;
    need = (size_t)kn_slices(w, cfg) * (size_t)rows * (size_t)w.n;
  }
  const int split = cfg ? cfg->split_k : 0;
  for (int t = 0; t < mfma2_tile_count(); ++t) {
    const size_t e = mfma2_partial_elems(w, batch, t, split);
    if (e > need) need = e;
  }
  return need;
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
        GemvNkFn f = w.fmt == kFmtBf16 ? gemv_nk_fn<kFmtBf16>(nb)
                     : w.fmt == kFmtExp ? gemv_nk_fn<kFmtExp>(nb) : gemv_nk_fn<kFmtPal>(nb);
        uint64_t blocks = (w.n + 3) / 4;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(256), 0, s, w, xb, nb, yb, ldy, col0);
      } else {
        const int slices = kn_slices(w, cfg);
        if (partial == nullptr || partial_elems < (size_t)slices * (size_t)nb * w.n) return hipErrorInvalidValue;
        const int64_t rows = (int64_t)((w.k + (uint64_t)slices - 1) / (uint64_t)slices);
        GemvKnFn f = w.fmt == kFmtBf16 ? gemv_kn_fn<kFmtBf16>(nb)
                     : w.fmt == kFmtExp ? gemv_kn_fn<kFmtExp>(nb) : gemv_kn_fn<kFmtPal>(nb);
        hipLaunchKernelGGL(f, dim3((unsigned)((w.n + 511) / 512), (unsigned)slices), dim3(256), 0, s, w, xb,
                           nb, partial, rows);
        uint64_t rb = ((uint64_t)nb * w.n + 255) / 256;
        if (rb > 4096) rb = 4096;
        hipLaunchKernelGGL(k_reduce_slices, dim3((unsigned)rb), dim3(256), 0, s, partial, slices, nb, w.n, yb,
                           ldy, col0);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_mfma2(w, x, batch, y, ldy, col0, v - 2, cfg ? cfg->split_k : 0, partial, partial_elems, s);
}

}  // namespace uw
