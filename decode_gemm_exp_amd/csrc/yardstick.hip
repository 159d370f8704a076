// yardstick.hip -- the achievable rates of the device, measured with this
// library's own kernels so the codec and GEMM figures can be read against
// them as well as against the published peaks:
//   * a streaming copy and a streaming read of HBM (each block a contiguous
//     span, 16-byte non-temporal vector accesses, four in flight per thread,
//     eight blocks per CU);
//   * an MFMA-only loop: v_mfma_f32_32x32x16_bf16 on register operands, four
//     independent accumulators per wave, two waves per SIMD on every CU, no
//     memory traffic.
// [EVC] "GPU記憶體瓶頸成關鍵" ("Cloudflare推出Unweight無損壓縮系統，將LLM模型大小
// 壓縮15-22%", easyvibecoding.app/curated/736): inference is bound by memory
// bandwidth, which is what the compressed formats trade arithmetic for; the
// copy and read kernels measure that bound on the box, the MFMA loop the
// other side of the roofline.
#include "uw_internal.h"

namespace uw {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Each block streams its own contiguous span, 16-byte vector accesses, four
// in flight per thread, non-temporal (read once, written once).  Of the read
// patterns measured on MI355X this one reads fastest: 6.7-6.8 TB/s on 1 GiB,
// against 6.0 for the same spans with cached loads and 5.2 for a grid-stride
// loop over the whole buffer.
__device__ __forceinline__ void span_of(uint64_t n16, uint64_t& b0, uint64_t& b1) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  b0 = (uint64_t)blockIdx.x * per;
  b1 = b0 + per < n16 ? b0 + per : n16;
  if (b0 > n16) b0 = n16;
}

__global__ __launch_bounds__(kThreads) void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                      uint64_t n16) {
  uint64_t b0, b1;
  span_of(n16, b0, b1);
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
  uint64_t i = b0 + threadIdx.x;
  for (; i + 3 * kThreads < b1; i += 4 * kThreads) {
    const u32x4_t a = __builtin_nontemporal_load(s + i), b = __builtin_nontemporal_load(s + i + kThreads),
                  c = __builtin_nontemporal_load(s + i + 2 * kThreads),
                  e = __builtin_nontemporal_load(s + i + 3 * kThreads);
    __builtin_nontemporal_store(a, d + i);
    __builtin_nontemporal_store(b, d + i + kThreads);
    __builtin_nontemporal_store(c, d + i + 2 * kThreads);
    __builtin_nontemporal_store(e, d + i + 3 * kThreads);
  }
  for (; i < b1; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

// Every thread folds what it read into one word and stores it, so no load can
// be dropped; the sink is one word per thread.
__global__ __launch_bounds__(kThreads) void k_read16(const uint4* __restrict__ src, uint64_t n16,
                                                      uint32_t* __restrict__ sink) {
  uint64_t b0, b1;
  span_of(n16, b0, b1);
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
  uint32_t acc = 0;
  uint64_t i = b0 + threadIdx.x;
  for (; i + 3 * kThreads < b1; i += 4 * kThreads) {
    const u32x4_t a = __builtin_nontemporal_load(s + i), b = __builtin_nontemporal_load(s + i + kThreads),
                  c = __builtin_nontemporal_load(s + i + 2 * kThreads),
                  e = __builtin_nontemporal_load(s + i + 3 * kThreads);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ e.x ^ e.y ^ e.z ^ e.w;
  }
  for (; i < b1; i += kThreads) {
    const u32x4_t a = __builtin_nontemporal_load(s + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Operands are non-zero and differ per lane (the matrix core's power, and the
// clock it holds, depend on the operand bits); the accumulators stay bounded
// because the B operands alternate in sign.
__global__ __launch_bounds__(kThreads) void k_mfma_loop(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b0, b1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.75f + 0.0078125f * (float)((lane * 7 + j * 3) & 31));
    b0[j] = (__bf16)(0.5f + 0.0039062f * (float)((lane * 5 + j) & 63));
    b1[j] = (__bf16)(-0.5f - 0.0039062f * (float)((lane * 3 + j * 5) & 63));
  }
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
  for (int64_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace uw

using namespace uw;

extern "C" uw_status uw_yardstick(int kind, const void* src_dev, void* dst_dev, size_t bytes, int64_t iters,
                                  void* stream, double* work) {
  if (!work || !dst_dev || (reinterpret_cast<uintptr_t>(dst_dev) & 15u)) return UW_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cus = device_cus();
  *work = 0;
  if (kind == 0 || kind == 1) {
    if (!src_dev || (reinterpret_cast<uintptr_t>(src_dev) & 15u) || bytes == 0 || bytes % 16 != 0)
      return UW_ERR_INVALID;
    const unsigned grid = (unsigned)cus * 8;
    if (kind == 0) {
      hipLaunchKernelGGL(k_copy16, dim3(grid), dim3(kThreads), 0, s, static_cast<const uint4*>(src_dev),
                         static_cast<uint4*>(dst_dev), (uint64_t)bytes / 16);
      *work = 2.0 * (double)bytes;
    } else {
      if ((size_t)grid * kThreads * 4 > UW_YARDSTICK_SINK_BYTES) return UW_ERR_UNSUPPORTED;
      hipLaunchKernelGGL(k_read16, dim3(grid), dim3(kThreads), 0, s, static_cast<const uint4*>(src_dev),
                         (uint64_t)bytes / 16, static_cast<uint32_t*>(dst_dev));
      *work = (double)bytes;
    }
  } else if (kind == 2) {
    if (iters <= 0) return UW_ERR_INVALID;
    const unsigned grid = (unsigned)cus * 2;   // two 4-wave blocks per CU: two waves per SIMD
    if ((size_t)grid * kThreads * 4 > UW_YARDSTICK_SINK_BYTES) return UW_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_mfma_loop, dim3(grid), dim3(kThreads), 0, s, iters, static_cast<float*>(dst_dev));
    *work = (double)grid * (kThreads / 64) * (double)iters * 4.0 * (2.0 * 32 * 32 * 16);
  } else {
    return UW_ERR_INVALID;
  }
  return hipGetLastError() == hipSuccess ? UW_OK : UW_ERR_DEVICE;
}
