// rebuild.h -- on-chip BF16 reconstruction shared by the decoder and the GEMM
// kernels.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "BF16權重壓縮原理": the weight
// is its sign bit, 8 exponent bits and 7 mantissa bits; section
// "重建矩陣乘法核心運作": the matmul joins exponent and sign+mantissa back
// into BF16 on chip.  Section "BF16權重壓縮原理" also fixes the verbatim
// rule: one flag per 64-weight group, tested once per group, never per weight.
//
// Byte-parallel forms (four weights per 32-bit operation):
//   * a BF16 weight is two bytes: lo = exponent bit 0 above the 7 mantissa
//     bits, hi = sign above exponent bits 7..1.  From 4 sign+mantissa bytes s
//     and 4 exponent bytes e, lo = bfi(0x80.., e << 7, s) and
//     hi = bfi(0x80.., s, e >> 1); two byte permutes interleave them into two
//     dwords of packed BF16 -- 6 VALU operations per 4 weights;
//   * 8 palette slots packed as nibbles (element i in nibble i) split into
//     even and odd elements with one mask each; a 16-entry palette is two
//     8-byte permute tables, the slot's bit 3 picks the table through a third
//     permute; a palette that is a run of consecutive exponents needs only a
//     bytewise add.  Two permutes restore element order.
#pragma once

#include "uw_internal.h"

namespace uw {

constexpr uint32_t kHiBits = 0x80808080u;

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (mask & a) | (~mask & b); }

// 4 sign+mantissa bytes + 4 exponent bytes -> 4 bf16 in two dwords
__device__ __forceinline__ void rebuild4(uint32_t s, uint32_t e, uint32_t& o0, uint32_t& o1) {
  const uint32_t lo = bfi(kHiBits, e << 7, s);
  const uint32_t hi = bfi(kHiBits, s, e >> 1);
  o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

__device__ __forceinline__ void rebuild16(const uint4& s, const uint4& e, uint32_t o[8]) {
  rebuild4(s.x, e.x, o[0], o[1]);
  rebuild4(s.y, e.y, o[2], o[3]);
  rebuild4(s.z, e.z, o[4], o[5]);
  rebuild4(s.w, e.w, o[6], o[7]);
}

// FP8 E4M3 weights (OCP OFP8 E4M3: sign bit 7, exponent bits 6..3, mantissa
// bits 2..0): 8 kept sign+mantissa nibbles (element i in bits 4i..4i+3,
// nibble = sign << 3 | mantissa) and the exponent fields of the same
// elements as bytes (e03: elements 0..3, e47: 4..7) -> 8 E4M3 bytes.
__device__ __forceinline__ void fp8_rebuild8(uint32_t nib, uint32_t e03, uint32_t e47, uint32_t& o03,
                                             uint32_t& o47) {
  const uint32_t ev = nib & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t od = (nib >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  const uint32_t s03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);
  const uint32_t s47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);
  o03 = ((s03 & 0x08080808u) << 4) | (e03 << 3) | (s03 & 0x07070707u);
  o47 = ((s47 & 0x08080808u) << 4) | (e47 << 3) | (s47 & 0x07070707u);
}

// 4 slot bytes (0..15) -> 4 palette exponent bytes
__device__ __forceinline__ uint32_t pal_lookup4(uint32_t n, const PalView& p) {
  const uint32_t n7 = n & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(p.w[1], p.w[0], n7);
  const uint32_t hi = __builtin_amdgcn_perm(p.w[3], p.w[2], n7);
  return __builtin_amdgcn_perm(hi, lo, ((n >> 1) & 0x04040404u) | 0x03020100u);
}

// 8 slots as nibbles (element i in bits 4i..4i+3) -> exponent bytes of
// elements 0..3 (e03) and 4..7 (e47); RUN: the palette is p.base4's entry
// onwards in steps of one
template <bool RUN>
__device__ __forceinline__ void pal8(uint32_t v, const PalView& p, uint32_t& e03, uint32_t& e47) {
  uint32_t ev = v & 0x0F0F0F0Fu;           // elements 0 2 4 6
  uint32_t od = (v >> 4) & 0x0F0F0F0Fu;    // elements 1 3 5 7
  if constexpr (RUN) {
    ev += p.base4;
    od += p.base4;
  } else {
    ev = pal_lookup4(ev, p);
    od = pal_lookup4(od, p);
  }
  e03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);
  e47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);
}

// 16 slots (two dwords of nibbles) -> 16 exponent bytes
template <bool RUN>
__device__ __forceinline__ uint4 pal16(uint32_t v0, uint32_t v1, const PalView& p) {
  uint4 e;
  pal8<RUN>(v0, p, e.x, e.y);
  pal8<RUN>(v1, p, e.z, e.w);
  return e;
}

// the same with the palette kind decided at run time (one uniform branch)
__device__ __forceinline__ uint4 pal16_any(uint32_t v0, uint32_t v1, const PalView& p) {
  return p.run ? pal16<true>(v0, v1, p) : pal16<false>(v0, v1, p);
}

// verbatim flag and rank of group g from its flag and rank words
__device__ __forceinline__ bool group_verbatim(uint32_t fw, uint64_t g) { return (fw >> (g & 31)) & 1u; }
__device__ __forceinline__ uint32_t group_rank(uint32_t fw, uint32_t rw, uint64_t g) {
  return rw + (uint32_t)__popc(fw & ((1u << (g & 31)) - 1u));
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
    if (group_verbatim(fw, g)) {   // verbatim group: exponents from the side section
      const uint32_t r = group_rank(fw, w.vrank[g >> 5], g);
      e = *reinterpret_cast<const uint4*>(w.vexp + (uint64_t)r * 64 + (el & 63));
    } else {
      e = pal16<FMT == kFmtPalRun>(nib.x, nib.y, w.pal);
    }
    rebuild16(s, e, o);
  }
}

// ---- chunk access shared by the pipelined GEMVs -------------------------------
// One chunk of OW (16 or 8) consecutive stored weights as loaded from HBM.
// Every load's address is known without waiting for another load: the
// palette format takes the chunk's verbatim flag word and rank word from an
// earlier pipeline step and then loads either the chunk's verbatim exponent
// bytes or the aligned index bytes that hold its OW nibbles.
template <int OW>
struct ChunkT {
  uint32_t a[OW / 2];   // bf16: the OW weights | exp, pal: OW sign+mantissa bytes in a[0 .. OW/4)
  uint32_t b[OW / 4];   // exp: OW exponent bytes | pal: 2*OW index nibbles or OW verbatim exponent bytes
};

// NT: a streaming (non-temporal) load, for weight data read once per call
template <int OW, bool NT = false>
__device__ __forceinline__ void load_words(const void* p, uint32_t* d) {   // OW / 4 dwords
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (OW == 16) {
    const u32x4_t v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p))
                         : *reinterpret_cast<const u32x4_t*>(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else {
    const u32x2_t v = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p))
                         : *reinterpret_cast<const u32x2_t*>(p);
    d[0] = v.x; d[1] = v.y;
  }
}

__device__ __forceinline__ uint32_t flag_index(uint64_t el) { return (uint32_t)(el >> 11); }

template <int FMT, int OW, bool NT = false>
__device__ __forceinline__ void chunk_load(const WeightView& w, uint64_t el, uint32_t fw, uint32_t rw, ChunkT<OW>& c) {
  if constexpr (FMT == kFmtBf16) {
    load_words<OW, NT>(w.bf16 + el, c.a);
    load_words<OW, NT>(w.bf16 + el + OW / 2, c.a + OW / 4);
  } else if constexpr (FMT == kFmtExp) {
    load_words<OW, NT>(w.sm + el, c.a);
    load_words<OW, NT>(w.ex + el, c.b);
  } else {
    load_words<OW, NT>(w.sm + el, c.a);
    const uint64_t g = el >> 6;
    const uint8_t* p = group_verbatim(fw, g) ? w.vexp + (uint64_t)group_rank(fw, rw, g) * 64 + (el & 63)
                                             : w.pidx + ((el >> 1) & ~(uint64_t)(OW - 1));
    load_words<OW, NT>(p, c.b);
  }
}

// OW / 2 dwords of packed bf16
template <int FMT, int OW>
__device__ __forceinline__ void chunk_rebuild(const WeightView& w, const ChunkT<OW>& c, uint64_t el, uint32_t fw,
                                              uint32_t* o) {
  if constexpr (FMT == kFmtBf16) {
#pragma unroll
    for (int i = 0; i < OW / 2; ++i) o[i] = c.a[i];
  } else {
    uint32_t e[OW / 4];
    if constexpr (FMT == kFmtExp) {
#pragma unroll
      for (int i = 0; i < OW / 4; ++i) e[i] = c.b[i];
    } else {
      const bool verb = group_verbatim(fw, el >> 6);
      if constexpr (OW == 16) {
        const bool hi = (el & 16) != 0;
        pal8<FMT == kFmtPalRun>(hi ? c.b[2] : c.b[0], w.pal, e[0], e[1]);
        pal8<FMT == kFmtPalRun>(hi ? c.b[3] : c.b[1], w.pal, e[2], e[3]);
      } else {
        pal8<FMT == kFmtPalRun>((el & 8) ? c.b[1] : c.b[0], w.pal, e[0], e[1]);
      }
#pragma unroll
      for (int i = 0; i < OW / 4; ++i) e[i] = verb ? c.b[i] : e[i];
    }
#pragma unroll
    for (int i = 0; i < OW / 4; ++i) rebuild4(c.a[i], e[i], o[2 * i], o[2 * i + 1]);
  }
}

template <int FMT>
__device__ __forceinline__ void flags_load(const WeightView& w, uint64_t el, uint32_t& fw, uint32_t& rw) {
  if constexpr (fmt_is_pal(FMT)) {
    fw = w.vflags[flag_index(el)];
    rw = w.vrank[flag_index(el)];
  } else {
    fw = rw = 0;
  }
}

__device__ __forceinline__ uint32_t wave_uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace uw
