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
// One wave per output row; each lane takes U chunks of 16 weights per pass
// (K positions lane*16 + u*1024), all loads of a pass issued before any use
// so that U x (compressed chunk) bytes per lane are in flight.
constexpr int kGemvU = 4;

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
// grid.x: blocks of 1024 outputs (64 lanes x 16); grid.y: K slices.  The 4
// waves of a block take rows kb + wave, kb + wave + 4, ...; each lane loads
// kGemvU rows' chunks before using any.  Every wave writes its own partial
// row part[slice * 4 + wave][b][n]; a second kernel adds them in fixed order.
template <int FMT, int NB>
__global__ __launch_bounds__(256) void k_gemv_kn(WeightView w, const uint16_t* __restrict__ x, int B,
                                                 float* __restrict__ part, int64_t rows_per_slice) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t N = w.n, K = w.k;
  const uint64_t n0 = (uint64_t)blockIdx.x * 1024 + (uint64_t)lane * 16;
  const uint64_t kb = (uint64_t)blockIdx.y * (uint64_t)rows_per_slice;
  const uint64_t ke = min(kb + (uint64_t)rows_per_slice, K);
  float acc[NB][16];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
  if (n0 < N) {
    for (uint64_t k0 = kb + (uint64_t)wave; k0 < ke; k0 += 4 * kGemvU) {
      uint32_t wv[kGemvU][8];
#pragma unroll
      for (int u = 0; u < kGemvU; ++u) {
        const uint64_t k = k0 + (uint64_t)u * 4;
        if (k < ke) {
          load16<FMT>(w, k * N + n0, wv[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) wv[u][i] = 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kGemvU; ++u) {
        const uint64_t k = k0 + (uint64_t)u * 4;
        if (k >= ke) break;
        float wf[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          wf[2 * i] = __uint_as_float(wv[u][i] << 16);
          wf[2 * i + 1] = __uint_as_float(wv[u][i] & 0xFFFF0000u);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b < B) {
            const float xb = __uint_as_float((uint32_t)x[(uint64_t)b * K + k] << 16);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][i] = fmaf(xb, wf[i], acc[b][i]);
          }
        }
      }
    }
  }
  if (n0 < N) {
    const uint64_t slot = (uint64_t)blockIdx.y * 4 + (uint64_t)wave;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < B) {
        float4* dst = reinterpret_cast<float4*>(part + (slot * (uint64_t)B + (uint64_t)b) * N + n0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[i] = make_float4(acc[b][4 * i], acc[b][4 * i + 1], acc[b][4 * i + 2], acc[b][4 * i + 3]);
      }
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

// K slices of the KN GEMV: enough blocks to cover the chip a few times
// (each slice at least 64 rows).
int kn_slices(const WeightView& w, const uw_kernel_cfg* cfg) {
  if (cfg && cfg->split_k > 0) return cfg->split_k;
  const uint64_t nblocks = (w.n + 1023) / 1024;
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

// Workspace floats for partial sums of the kernel this call resolves to (the
// KN GEMV's K slices or the MFMA split-K slices).
size_t gemm_partial_elems(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg) {
  const int v = resolve_variant(w, batch, cfg);
  if (v == 1) {
    if (w.layout == 0) return 0;
    const int64_t rows = batch < kGemvMaxBatch ? batch : kGemvMaxBatch;
    return 4 * (size_t)kn_slices(w, cfg) * (size_t)rows * (size_t)w.n;
  }
  return mfma2_partial_elems(w, batch, v - 2, cfg ? cfg->split_k : 0);
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
        if (partial == nullptr || partial_elems < 4 * (size_t)slices * (size_t)nb * w.n) return hipErrorInvalidValue;
        const int64_t rows = (int64_t)((w.k + (uint64_t)slices - 1) / (uint64_t)slices);
        GemvKnFn f = w.fmt == kFmtBf16 ? gemv_kn_fn<kFmtBf16>(nb)
                     : w.fmt == kFmtExp ? gemv_kn_fn<kFmtExp>(nb) : gemv_kn_fn<kFmtPal>(nb);
        hipLaunchKernelGGL(f, dim3((unsigned)((w.n + 1023) / 1024), (unsigned)slices), dim3(256), 0, s, w, xb,
                           nb, partial, rows);
        uint64_t rb = ((uint64_t)nb * w.n + 255) / 256;
        if (rb > 4096) rb = 4096;
        hipLaunchKernelGGL(k_reduce_slices, dim3((unsigned)rb), dim3(256), 0, s, partial, 4 * slices, nb, w.n, yb,
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
