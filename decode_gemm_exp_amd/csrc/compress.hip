// compress.hip -- GPU passes of uw_compress on gfx950.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736), section "BF16權重壓縮原理": sign and
// mantissa kept, exponent byte entropy-coded, top-16 exponent palette, a
// 64-weight row with an out-of-palette exponent kept verbatim after one
// check per row.
//
// Passes (all memory-bound, each one sweep over the weights):
//   histogram     256-bin exponent counts, privatised per wave in LDS
//   flags         per 64-weight group: any exponent outside the palette
//                 (wave ballot), sign+mantissa bytes, coded-slot histogram
//   rank scan     exclusive prefix of popcount(vflags) (multi-block scan)
//   segment bits  code bits per segment -> words per segment
//   offsets scan  exclusive prefix of words -> seg_off
//   encode        one wave per segment: per-lane codeword, wave prefix sum of
//                 lengths gives bit positions, LDS atomic-or packs the words;
//                 verbatim groups copy their exponents to the side section.
//
// FP8 E4M3 weights (UWF8 reading of saidapartage.blog, "Cloudflare Unweight :
// -22 % sur le poids de vos LLM, sans perdre un bit", section "Un complément,
// pas un remplaçant": the coding also applies on top of quantisation): two
// more passes put each weight's 4-bit exponent field where a BF16 exponent
// byte sits, so the passes above code it unchanged, and pack the kept
// sign+mantissa nibbles two per byte.
#include "uw_internal.h"

namespace uw {
namespace {

__device__ __forceinline__ uint32_t exp_of(uint32_t b) { return (b >> 7) & 0xFFu; }
__device__ __forceinline__ uint32_t sm_of(uint32_t b) { return ((b >> 8) & 0x80u) | (b & 0x7Fu); }

// ---- histogram ----------------------------------------------------------------
__global__ __launch_bounds__(256) void k_histogram(const uint4* __restrict__ w, uint64_t n8,
                                                   uint32_t* __restrict__ hist) {
  // 16 copies indexed by lane % 16: the few hot exponents of a weight matrix
  // would otherwise serialise 64 lanes on one LDS word
  __shared__ uint32_t h[16][256];
  const int copy = threadIdx.x & 15;
  for (int i = threadIdx.x; i < 16 * 256; i += 256) (&h[0][0])[i] = 0;
  __syncthreads();
  for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n8; i += (uint64_t)gridDim.x * 256ull) {
    uint4 v = w[i];
    uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      atomicAdd(&h[copy][exp_of(d[j] & 0xFFFFu)], 1u);
      atomicAdd(&h[copy][exp_of(d[j] >> 16)], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 256; i += 256) {
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) s += h[c][i];
    if (s) atomicAdd(&hist[i], s);
  }
}

// ---- flags + sign/mantissa + coded histogram ------------------------------------
// One wave per 32 groups (one flag word): four rounds of 8 groups, 8 lanes per
// group, 8 weights (16 bytes) per lane.
__global__ __launch_bounds__(256) void k_flags(const uint4* __restrict__ w, uint64_t groups,
                                               const uint8_t* __restrict__ slot_tab,
                                               uint2* __restrict__ sm, uint32_t* __restrict__ vflags,
                                               uint32_t* __restrict__ coded) {
  __shared__ int8_t slot[256];
  __shared__ uint32_t cnt[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 256; i += 256) slot[i] = (int8_t)slot_tab[i];
  if (threadIdx.x < 64) (&cnt[0][0])[threadIdx.x] = 0;
  __syncthreads();
  const uint64_t nwords = (groups + 31) / 32;
  for (uint64_t word = blockIdx.x * 4ull + wave; word < nwords; word += (uint64_t)gridDim.x * 4ull) {
    uint32_t flagword = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint64_t g = word * 32 + (uint64_t)r * 8 + (uint64_t)(lane >> 3);
      const bool valid = g < groups;
      bool outside = false;
      int s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (valid) {
        const uint64_t e8 = g * 8 + (uint64_t)(lane & 7);   // index in units of 8 weights
        uint4 v = w[e8];
        uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t smw[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t b = (j & 1) ? (d[j >> 1] >> 16) : (d[j >> 1] & 0xFFFFu);
          s[j] = slot[exp_of(b)];
          outside |= s[j] < 0;
          smw[j >> 2] |= sm_of(b) << (8 * (j & 3));
        }
        sm[e8] = make_uint2(smw[0], smw[1]);
      }
      const uint64_t ball = __ballot(outside);
      const bool verbatim = ((ball >> (lane & ~7)) & 0xFFull) != 0;
      // flag bits for the 8 groups of this round
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if ((ball >> (8 * q)) & 0xFFull) flagword |= 1u << (r * 8 + q);
      if (valid && !verbatim) {
#pragma unroll
        for (int j = 0; j < 8; ++j) atomicAdd(&cnt[wave][s[j]], 1u);
      }
    }
    if (lane == 0) vflags[word] = flagword;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    uint32_t c = cnt[0][threadIdx.x] + cnt[1][threadIdx.x] + cnt[2][threadIdx.x] + cnt[3][threadIdx.x];
    if (c) atomicAdd(&coded[threadIdx.x], c);
  }
}

// ---- exclusive scans --------------------------------------------------------------
// Block-wide exclusive scan of one value per thread (1024 threads).
__device__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* total) {
  __shared__ uint64_t wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint64_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t run = 0;
    for (int i = 0; i < 16; ++i) {
      uint64_t t = wsum[i];
      wsum[i] = run;
      run += t;
    }
    *total = run;
  }
  __syncthreads();
  uint64_t r = wsum[wave] + x - v;
  __syncthreads();
  return r;
}

// Multi-block exclusive scan of n u32 values (or their popcounts), 64-bit
// running sums: tile sums, a one-block scan of the tile sums, then each tile
// scans itself from its offset.  A tile is 1024 threads x 8 values.
constexpr int kScanPer = 8;
constexpr uint64_t kScanTile = 1024ull * kScanPer;

template <bool POPC>
__device__ __forceinline__ uint64_t scan_in(const uint32_t* in, uint64_t i, uint64_t n) {
  if (i >= n) return 0;
  const uint32_t v = in[i];
  return POPC ? (uint64_t)__popc(v) : (uint64_t)v;
}

template <bool POPC>
__global__ __launch_bounds__(1024) void k_scan_tiles(const uint32_t* __restrict__ in, uint64_t n,
                                                     uint64_t* __restrict__ sums) {
  __shared__ uint64_t tot;
  const uint64_t base = (uint64_t)blockIdx.x * kScanTile;
  uint64_t s = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) s += scan_in<POPC>(in, base + (uint64_t)j * 1024 + threadIdx.x, n);
  (void)block_exclusive_scan(s, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

__global__ __launch_bounds__(1024) void k_scan_sums(uint64_t* __restrict__ sums, uint64_t tiles,
                                                    uint64_t* __restrict__ total, uint32_t* __restrict__ total32) {
  __shared__ uint64_t chunk_total;
  uint64_t carry = 0;
  for (uint64_t base = 0; base < tiles; base += 1024) {
    const uint64_t i = base + threadIdx.x;
    const uint64_t v = i < tiles ? sums[i] : 0;
    const uint64_t ex = block_exclusive_scan(v, &chunk_total);
    if (i < tiles) sums[i] = carry + ex;
    __syncthreads();
    carry += chunk_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (total) *total = carry;
    if (total32) *total32 = (uint32_t)carry;
  }
}

template <bool POPC>
__global__ __launch_bounds__(1024) void k_scan_apply(const uint32_t* __restrict__ in, uint64_t n,
                                                     const uint64_t* __restrict__ offs, uint32_t* __restrict__ out) {
  __shared__ uint64_t tot;
  const uint64_t base = (uint64_t)blockIdx.x * kScanTile + (uint64_t)threadIdx.x * kScanPer;
  uint64_t v[kScanPer];
  uint64_t s = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    v[j] = scan_in<POPC>(in, base + j, n);
    s += v[j];
  }
  uint64_t run = offs[blockIdx.x] + block_exclusive_scan(s, &tot);
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    if (base + j < n) out[base + j] = (uint32_t)run;
    run += v[j];
  }
}

template <bool POPC>
hipError_t scan3(const uint32_t* in, uint64_t n, uint32_t* out, uint64_t* total, uint32_t* total32, uint64_t* tiles_ws,
                 hipStream_t s) {
  const uint64_t tiles = (n + kScanTile - 1) / kScanTile;
  if (tiles == 0 || tiles > 0x7FFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_scan_tiles<POPC>, dim3((unsigned)tiles), dim3(1024), 0, s, in, n, tiles_ws);
  hipLaunchKernelGGL(k_scan_sums, dim3(1), dim3(1024), 0, s, tiles_ws, tiles, total, total32);
  hipLaunchKernelGGL(k_scan_apply<POPC>, dim3((unsigned)tiles), dim3(1024), 0, s, in, n, tiles_ws, out);
  return hipGetLastError();
}

// ---- per-segment code bits -------------------------------------------------------
// One wave per 8 groups (8 lanes x 8 weights per group).  Group bit counts are
// summed per segment with an atomic add (segments are <= 64 groups).
__global__ __launch_bounds__(256) void k_segment_bits(const uint4* __restrict__ w, uint64_t groups,
                                                      uint32_t seg_groups, const uint8_t* __restrict__ len_tab,
                                                      const uint32_t* __restrict__ vflags,
                                                      uint32_t* __restrict__ seg_bits) {
  __shared__ uint8_t len[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 256; i += 256) len[i] = len_tab[i];
  __syncthreads();
  const uint64_t rounds = (groups + 7) / 8;
  for (uint64_t r = blockIdx.x * 4ull + wave; r < rounds; r += (uint64_t)gridDim.x * 4ull) {
    const uint64_t g = r * 8 + (uint64_t)(lane >> 3);
    uint32_t bits = 0;
    if (g < groups && !((vflags[g >> 5] >> (g & 31)) & 1u)) {
      uint4 v = w[g * 8 + (uint64_t)(lane & 7)];
      uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) bits += len[exp_of(d[j] & 0xFFFFu)] + len[exp_of(d[j] >> 16)];
    }
    // reduce over the 8 lanes of a group
    bits += __shfl_xor(bits, 1, 64);
    bits += __shfl_xor(bits, 2, 64);
    bits += __shfl_xor(bits, 4, 64);
    if ((lane & 7) == 0 && g < groups && bits) atomicAdd(&seg_bits[g / seg_groups], bits);
  }
}

__global__ void k_bits_to_words(uint32_t* __restrict__ v, uint64_t n) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    v[i] = (v[i] + 31u) >> 5;
}

// ---- encoder ------------------------------------------------------------------------
// One wave per segment.  Lane j codes weight j of each group; an inclusive
// wave scan of code lengths places every codeword; LDS atomic-or assembles
// the segment's words (<= 64 groups x 64 x 12 bits = 1536 words), which are
// then copied out.  codebook[e] = (code << 8) | len for palette exponents.
constexpr int kEncWaves = 4;
constexpr int kEncMaxWords = 64 * 64 * kMaxLen / 32;

__global__ __launch_bounds__(256) void k_encode(const uint16_t* __restrict__ w, uint64_t groups,
                                                uint32_t seg_groups, uint64_t segments,
                                                const uint32_t* __restrict__ codebook,
                                                const uint32_t* __restrict__ vflags,
                                                const uint32_t* __restrict__ vrank,
                                                const uint32_t* __restrict__ seg_off,
                                                uint32_t* __restrict__ stream, uint8_t* __restrict__ vexp) {
  __shared__ uint32_t book[256];
  __shared__ uint32_t words[kEncWaves][kEncMaxWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 256; i += 256) book[i] = codebook[i];
  __syncthreads();
  for (uint64_t s = blockIdx.x * (uint64_t)kEncWaves + wave; s < segments;
       s += (uint64_t)gridDim.x * kEncWaves) {
    const uint32_t w0 = seg_off[s], nw = seg_off[s + 1] - w0;
    for (uint32_t i = lane; i < nw; i += 64) words[wave][i] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint32_t bitbase = 0;
    const uint64_t g0 = s * seg_groups;
    const uint64_t g1 = min(g0 + seg_groups, groups);
    // a segment's groups share one flag word (segments are <= 32 groups or
    // whole words); weights are loaded four groups ahead of their coding
    uint32_t bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[q] = g0 + q < g1 ? w[(g0 + q) * 64 + (uint64_t)lane] : 0u;
    for (uint64_t g = g0; g < g1; ++g) {
      const uint32_t fw = vflags[g >> 5];
      const uint32_t b = bq[0];
      bq[0] = bq[1];
      bq[1] = bq[2];
      bq[2] = bq[3];
      bq[3] = g + 4 < g1 ? w[(g + 4) * 64 + (uint64_t)lane] : 0u;
      const uint32_t e = exp_of(b);
      if ((fw >> (g & 31)) & 1u) {
        const uint32_t rank = vrank[g >> 5] + (uint32_t)__popc(fw & ((1u << (g & 31)) - 1u));
        vexp[(uint64_t)rank * 64 + (uint64_t)lane] = (uint8_t)e;
        continue;
      }
      const uint32_t cw = book[e];
      const uint32_t len = cw & 0xFFu, code = cw >> 8;
      uint32_t incl = len;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
      }
      const uint32_t pos = bitbase + incl - len;     // first bit of this codeword
      const uint32_t wi = pos >> 5, off = pos & 31u;
      // codeword occupies bits [off, off+len) counted from the word's MSB
      if (off + len <= 32) {
        atomicOr(&words[wave][wi], code << (32 - off - len));
      } else {
        const uint32_t spill = off + len - 32;
        atomicOr(&words[wave][wi], code >> spill);
        atomicOr(&words[wave][wi + 1], code << (32 - spill));
      }
      bitbase += __shfl(incl, 63, 64);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (uint32_t i = lane; i < nw; i += 64) stream[w0 + i] = words[wave][i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

// Largest stream span of any decoder wave (64 consecutive segments), counted
// from the 4-word boundary below its first word: sizes the decoder's LDS copy.
__global__ __launch_bounds__(256) void k_wave_span(const uint32_t* __restrict__ seg_off, uint64_t segments,
                                                   uint32_t* __restrict__ out) {
  const uint64_t waves = (segments + 63) / 64;
  for (uint64_t w = blockIdx.x * 256ull + threadIdx.x; w < waves; w += (uint64_t)gridDim.x * 256ull) {
    const uint64_t e = min((w + 1) * 64, segments);
    const uint32_t span = seg_off[e] - (seg_off[w * 64] & ~3u);
    atomicMax(out, span);
  }
}

// ---- FP8 E4M3 field passes (16 weights per thread and step) --------------------
// exponent field (bits 6..3) -> bits 14..7 of a 16-bit word, all else zero
__global__ __launch_bounds__(256) void k_fp8_fields(const uint4* __restrict__ w, uint64_t n16,
                                                    uint4* __restrict__ out) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint4 v = w[i];
    const uint32_t src[4] = {v.x, v.y, v.z, v.w};
    uint32_t dst[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = (src[j] >> 3) & 0x0F0F0F0Fu;   // byte b holds element 4j+b's field
      dst[2 * j] = ((e & 0xFFu) << 7) | (((e >> 8) & 0xFFu) << 23);
      dst[2 * j + 1] = (((e >> 16) & 0xFFu) << 7) | ((e >> 24) << 23);
    }
    out[2 * i] = make_uint4(dst[0], dst[1], dst[2], dst[3]);
    out[2 * i + 1] = make_uint4(dst[4], dst[5], dst[6], dst[7]);
  }
}

// sign << 3 | mantissa per weight, element 2i in the low nibble of byte i
__global__ __launch_bounds__(256) void k_fp8_pack(const uint4* __restrict__ w, uint64_t n16,
                                                  uint2* __restrict__ out) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const uint4 v = w[i];
    const uint32_t src[4] = {v.x, v.y, v.z, v.w};
    uint32_t half[4];   // 16 bits: the nibbles of 4 weights
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t nib = ((src[j] >> 4) & 0x08080808u) | (src[j] & 0x07070707u);   // byte b: element 4j+b
      half[j] = (nib & 0xFu) | (((nib >> 8) & 0xFu) << 4) | (((nib >> 16) & 0xFu) << 8) | ((nib >> 24) << 12);
    }
    out[i] = make_uint2(half[0] | (half[1] << 16), half[2] | (half[3] << 16));
  }
}

unsigned grid_for(uint64_t items, unsigned per_block, unsigned cap = 65535u * 4u) {
  uint64_t b = (items + per_block - 1) / per_block;
  if (b == 0) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_fp8_fields(const uint8_t* w, uint64_t numel, uint16_t* out, hipStream_t s) {
  const uint64_t n16 = numel / 16;   // numel is a multiple of 64
  hipLaunchKernelGGL(k_fp8_fields, dim3(grid_for(n16, 256 * 4, 8192)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w), n16, reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_fp8_pack(const uint8_t* w, uint64_t numel, uint8_t* out, hipStream_t s) {
  const uint64_t n16 = numel / 16;
  hipLaunchKernelGGL(k_fp8_pack, dim3(grid_for(n16, 256 * 4, 8192)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w), n16, reinterpret_cast<uint2*>(out));
  return hipGetLastError();
}

hipError_t launch_histogram(const uint16_t* w, uint64_t numel, uint32_t* hist, hipStream_t s) {
  const uint64_t n8 = numel / 8;   // numel is a multiple of 64
  hipLaunchKernelGGL(k_histogram, dim3(grid_for(n8, 256 * 8, 2048)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w), n8, hist);
  return hipGetLastError();
}

hipError_t launch_flags(const uint16_t* w, uint64_t numel, uint64_t groups, const uint8_t* slot_tab,
                        uint8_t* sm, uint32_t* vflags, uint32_t* coded, hipStream_t s) {
  (void)numel;
  const uint64_t words = (groups + 31) / 32;
  hipLaunchKernelGGL(k_flags, dim3(grid_for(words, 4 * 4, 8192)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w), groups, slot_tab,
                     reinterpret_cast<uint2*>(sm), vflags, coded);
  return hipGetLastError();
}

hipError_t launch_rank_scan(const uint32_t* vflags, uint64_t words, uint32_t* vrank, uint64_t* total,
                            uint64_t* tiles_ws, hipStream_t s) {
  return scan3<true>(vflags, words, vrank, total, nullptr, tiles_ws, s);
}

hipError_t launch_segment_bits(const uint16_t* w, uint64_t groups, uint32_t seg_groups, uint64_t segments,
                               const uint8_t* len_tab, const uint32_t* vflags, uint32_t* seg_words,
                               hipStream_t s) {
  const uint64_t rounds = (groups + 7) / 8;
  hipLaunchKernelGGL(k_segment_bits, dim3(grid_for(rounds, 4 * 8, 8192)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w), groups, seg_groups, len_tab, vflags, seg_words);
  hipLaunchKernelGGL(k_bits_to_words, dim3(grid_for(segments, 256 * 4, 4096)), dim3(256), 0, s,
                     seg_words, segments);
  return hipGetLastError();
}

hipError_t launch_offsets_scan(const uint32_t* seg_words, uint64_t segments, uint32_t* seg_off,
                               uint64_t* tiles_ws, hipStream_t s) {
  return scan3<false>(seg_words, segments, seg_off, nullptr, seg_off + segments, tiles_ws, s);
}

uint64_t scan_tiles(uint64_t n) { return (n + kScanTile - 1) / kScanTile; }

hipError_t launch_wave_span(const uint32_t* seg_off, uint64_t segments, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_wave_span, dim3(grid_for((segments + 63) / 64, 256, 1024)), dim3(256), 0, s, seg_off,
                     segments, out);
  return hipGetLastError();
}

hipError_t launch_encode(const uint16_t* w, uint64_t groups, uint32_t seg_groups, uint64_t segments,
                         const uint32_t* codebook, const uint32_t* vflags, const uint32_t* vrank,
                         const uint32_t* seg_off, uint32_t* stream, uint8_t* vexp, hipStream_t s) {
  hipLaunchKernelGGL(k_encode, dim3(grid_for(segments, kEncWaves, 16384)), dim3(256), 0, s, w, groups,
                     seg_groups, segments, codebook, vflags, vrank, seg_off, stream, vexp);
  return hipGetLastError();
}

}  // namespace uw
