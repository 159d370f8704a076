// rebuild.h -- on-chip BF16 reconstruction shared by the GEMM kernels.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "BF16權重壓縮原理": the weight
// is its sign bit, 8 exponent bits and 7 mantissa bits; section
// "重建矩陣乘法核心運作": the matmul joins exponent and sign+mantissa back
// into BF16 on chip.  Section "BF16權重壓縮原理" also fixes the verbatim
// rule: one flag per 64-weight group, tested once per group, never per weight.
#pragma once

#include "uw_internal.h"

namespace uw {

// 4 nibbles (low 16 bits) -> 4 bytes, byte i = nibble i
__device__ __forceinline__ uint32_t nib_spread(uint32_t v) {
  uint32_t x = v & 0xFFFFu;
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  return x;
}

// 4 slot bytes -> 4 palette exponent bytes (v_perm over the 16 palette bytes)
__device__ __forceinline__ uint32_t pal_lookup(uint32_t sel, const uint32_t* pal) {
  const uint32_t s7 = sel & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(pal[1], pal[0], s7);
  const uint32_t hi = __builtin_amdgcn_perm(pal[3], pal[2], s7);
  const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xFFu;
  return (hi & m) | (lo & ~m);
}

// interleaved bytes [s0 e0 s1 e1] -> two packed bf16
__device__ __forceinline__ uint32_t rebuild_pair(uint32_t x) {
  uint32_t r = (x & 0x007F007Fu) | ((x >> 1) & 0x7F807F80u);
  return r | ((x << 8) & 0x80008000u);
}

// 4 sign+mantissa bytes + 4 exponent bytes -> 4 bf16 in two dwords
__device__ __forceinline__ void rebuild4(uint32_t s, uint32_t e, uint32_t& o0, uint32_t& o1) {
  o0 = rebuild_pair(__builtin_amdgcn_perm(e, s, 0x05010400u));
  o1 = rebuild_pair(__builtin_amdgcn_perm(e, s, 0x07030602u));
}

__device__ __forceinline__ void rebuild16(const uint4& s, const uint4& e, uint32_t o[8]) {
  rebuild4(s.x, e.x, o[0], o[1]);
  rebuild4(s.y, e.y, o[2], o[3]);
  rebuild4(s.z, e.z, o[4], o[5]);
  rebuild4(s.w, e.w, o[6], o[7]);
}

// 16 consecutive stored weights starting at stored index `el` (el % 16 == 0)
// -> 8 dwords of packed bf16, for each weight format.
template <int FMT>
__device__ __forceinline__ void load16(const WeightView& w, uint64_t el, uint32_t o[8]) {
  if constexpr (FMT == kFmtBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(w.bf16 + el);
    const uint4 a = p[0], b = p[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  } else if constexpr (FMT == kFmtExp) {
    const uint4 s = *reinterpret_cast<const uint4*>(w.sm + el);
    const uint4 e = *reinterpret_cast<const uint4*>(w.ex + el);
    rebuild16(s, e, o);
  } else {
    const uint4 s = *reinterpret_cast<const uint4*>(w.sm + el);
    const uint2 nib = *reinterpret_cast<const uint2*>(w.pidx + el / 2);
    const uint64_t g = el >> 6;
    const uint32_t fw = w.vflags[g >> 5];
    uint4 e;
    if ((fw >> (g & 31)) & 1u) {   // verbatim group: exponents from the side section
      const uint32_t r = w.vrank[g >> 5] + (uint32_t)__popc(fw & ((1u << (g & 31)) - 1u));
      e = *reinterpret_cast<const uint4*>(w.vexp + (uint64_t)r * 64 + (el & 63));
    } else {
      e.x = pal_lookup(nib_spread(nib.x), w.pal);
      e.y = pal_lookup(nib_spread(nib.x >> 16), w.pal);
      e.z = pal_lookup(nib_spread(nib.y), w.pal);
      e.w = pal_lookup(nib_spread(nib.y >> 16), w.pal);
    }
    rebuild16(s, e, o);
  }
}

// 8 consecutive stored weights at `el` (el % 8 == 0) -> 4 dwords of bf16
template <int FMT>
__device__ __forceinline__ void load8(const WeightView& w, uint64_t el, uint32_t o[4]) {
  if constexpr (FMT == kFmtBf16) {
    const uint4 a = *reinterpret_cast<const uint4*>(w.bf16 + el);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  } else if constexpr (FMT == kFmtExp) {
    const uint2 s = *reinterpret_cast<const uint2*>(w.sm + el);
    const uint2 e = *reinterpret_cast<const uint2*>(w.ex + el);
    rebuild4(s.x, e.x, o[0], o[1]);
    rebuild4(s.y, e.y, o[2], o[3]);
  } else {
    const uint2 s = *reinterpret_cast<const uint2*>(w.sm + el);
    const uint32_t nib = *reinterpret_cast<const uint32_t*>(w.pidx + el / 2);
    const uint64_t g = el >> 6;
    const uint32_t fw = w.vflags[g >> 5];
    uint2 e;
    if ((fw >> (g & 31)) & 1u) {
      const uint32_t r = w.vrank[g >> 5] + (uint32_t)__popc(fw & ((1u << (g & 31)) - 1u));
      e = *reinterpret_cast<const uint2*>(w.vexp + (uint64_t)r * 64 + (el & 63));
    } else {
      e.x = pal_lookup(nib_spread(nib), w.pal);
      e.y = pal_lookup(nib_spread(nib >> 16), w.pal);
    }
    rebuild4(s.x, e.x, o[0], o[1]);
    rebuild4(s.y, e.y, o[2], o[3]);
  }
}

}  // namespace uw
