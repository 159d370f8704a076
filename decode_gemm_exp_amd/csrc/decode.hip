// decode.hip -- chunked-bitstream Huffman decoder for gfx950, four outputs:
//   nibble   : 4-bit palette indices (palette transcode)
//   exponent : exponent bytes (exponent-only decode)
//   full     : rebuilt BF16 (full decode)
//   fp8      : rebuilt E4M3 bytes (FP8 handles: exponent fields + kept nibbles)
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736): section "四種執行管道" defines the
// three preprocessing outputs; section "解壓與運算資源共享" gives the
// decoder a 16 KB lookup table in on-chip memory; this kernel keeps a 32 KB
// one in LDS (4096 two-word entries, up to eight codewords per window).
//
// Work split.  One lane owns one segment (seg_groups consecutive groups whose
// codes start on a word boundary), so every lane knows where its output goes
// without any search.
//
// Decode loop (per lane).  A 64-bit MSB-aligned bit buffer is fed from a
// queue of three prefetched 16-byte stream chunks (raw buffer loads: reads
// past the stream return zero instead of faulting), so a chunk is requested
// about 8 words before it is needed.  Each step refills 32 bits if fewer than
// 24 remain and then looks up two 12-bit windows in the LDS table; an entry
// gives up to eight whole codewords (their palette slots as nibbles) and their
// total length.  Slots accumulate in a 16-nibble register and leave 8 at a
// time into the wave's LDS stage.  A lane decodes all coded groups of a round
// (up to 8 groups) in one loop, so lanes only meet at the end of a round.
//
// Copy-out (per wave, every lane active).  The 64 segments of a wave write a
// contiguous output range, swept 16 weights per lane per step: 16-byte
// coalesced stores, verbatim groups taken from the side section, the palette
// lookup (v_perm over the 16 palette bytes) and the BF16 rebuild done here.
// The owner lane's verbatim flags and rank reach the copying lane through a
// cross-lane shuffle.  Stage word f of lane L sits at f * 64 + (L ^ f), which
// keeps both the per-lane writes and the per-owner reads on distinct banks.
#include <cstdlib>

#include "rebuild.h"

namespace uw {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRound = 8;                      // groups per decode round
constexpr int kStageWords = kRound * 8;        // 8 slot nibbles per word, 64 per group

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// 16 bytes of the coded stream.  NT: a non-temporal load, for the transcode
// (read once, front to back: 8B gate 26.7 -> 24.9 us, 70B gate 98.2 -> 91.4
// us); the exponent decode ran 3 % slower with it and the full decode the
// same, so they keep cached loads.
template <bool NT = false>
__device__ __forceinline__ uint4 load_chunk(__amdgpu_buffer_rsrc_t r, uint32_t word) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(word * 4u), 0, NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// byte-addressed raw buffer accesses: an offset at or past the resource's
// end reads zero and drops the write
constexpr uint32_t kPastEnd = 0x7FFF0000u;    // offset past every resource below
constexpr uint32_t kRecordsMax = 0x40000000u; // resources span at most 1 GiB
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Cache policy of the 16-byte output stores.  NT (non-temporal) streams
// data written once to HBM: exponent decode on the 8B gate 37 -> 31 us with
// outputs rotating over more than the 256 MB last-level cache, 33 -> 31 us
// with one output buffer reused per call.  The full decode's BF16 output is
// read back by the GEMM right after it; while it fits in half of that cache
// a reused buffer stays there and cached stores win (49 vs 54 us on the 8B
// gate), above that NT wins (rotated: 56 -> 52 us).  The transcode's 8-byte
// stores always stay cached: L2 merges the two halves of each 16-byte piece,
// as NT stores they took 26 -> 42 us.
constexpr int kCachePolicyNT = 2;
constexpr uint64_t kCachedOutputMax = 128ull << 20;
template <bool NT>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t byte, uint4 d) {
  u32x4 v = {d.x, d.y, d.z, d.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte, 0, NT ? kCachePolicyNT : 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t byte, uint32_t lo, uint32_t hi) {
  u32x2 v = {lo, hi};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)byte, 0, 0);
}
// output bytes before weight el: 4-bit slots, exponent bytes or BF16
template <int MODE>
__device__ __forceinline__ uint64_t out_bytes(uint64_t el) {
  return MODE == kDecodeNibble ? el >> 1 : (MODE == kDecodeExponent || MODE == kDecodeFp8) ? el : el * 2u;
}

__device__ __forceinline__ uint32_t stage_at(uint32_t f, uint32_t L) { return f * 64u + (L ^ (f & 63u)); }

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_decode_direct(DecodeArgs a) {
  __shared__ uint2 lut[1 << kLutBits];
  __shared__ uint32_t stage_all[kWaves][64 * kStageWords];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* stage = stage_all[wave];

  const uint64_t sbase = (uint64_t)blockIdx.x * kThreads + (uint64_t)wave * 64;
  const uint64_t s = sbase + (uint64_t)lane;
  const bool sval = s < a.segments;
  const uint32_t SG = a.seg_groups;
  const uint32_t CH = SG < (uint32_t)kRound ? SG : (uint32_t)kRound;   // groups per round
  const uint32_t rounds = SG / CH;
  // segment bounds first, so their latency overlaps the table load
  const uint32_t w0 = sval ? a.seg_off[s] : 0u;
  const uint32_t w1 = sval ? a.seg_off[s + 1] : 0u;

  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.stream, (short)0, (int)(a.stream_words * 4u), 0x00020000);
  uint32_t cw = w0 & ~3u, qi = w0 & 3u;
  uint4 q0 = load_chunk(rs, cw);
  uint4 q1 = load_chunk(rs, cw + 4);
  uint4 q2 = load_chunk(rs, cw + 8);

  for (int i = threadIdx.x; i < (1 << kLutBits); i += kThreads) lut[i] = reinterpret_cast<const uint2*>(a.lut)[i];
  __syncthreads();

  uint64_t buf = 0;
  int avail = 0;
  uint32_t consumed = 0;
  bool bad = false;
  auto refill = [&]() {
    const uint32_t word = qi == 0 ? q0.x : qi == 1 ? q0.y : qi == 2 ? q0.z : q0.w;
    buf |= (uint64_t)word << (32 - avail);
    avail += 32;
    if (++qi == 4) {
      q0 = q1;
      q1 = q2;
      qi = 0;
      cw += 4;
      q2 = load_chunk(rs, cw + 8);
    }
  };
  refill();
  refill();

  uint64_t acc = 0;     // pending slot nibbles, first decoded in the low nibble
  int n = 0;
  uint32_t coded_groups = 0;
  const PalView pal = a.pal;
  const uint8_t* __restrict__ vexp = a.vexp;
  const uint8_t* __restrict__ smp = a.sm;

  for (uint32_t r = 0; r < rounds; ++r) {
    // verbatim flags and rank of this lane's groups in the round (<= 8 groups,
    // always inside one 32-group flag word)
    const uint64_t g0 = s * SG + (uint64_t)r * CH;
    uint32_t vbits = 0, rank0 = 0, ngroups = 0;
    if (sval && g0 < a.groups) {
      const uint32_t fw = a.vflags[g0 >> 5];
      const uint32_t sh = (uint32_t)(g0 & 31);
      const uint64_t left = a.groups - g0;
      ngroups = left < CH ? (uint32_t)left : CH;
      vbits = (fw >> sh) & ((1u << ngroups) - 1u);
      rank0 = a.vrank[g0 >> 5] + (uint32_t)__popc(fw & ((1u << sh) - 1u));
    }
    const uint32_t ncoded = ngroups - (uint32_t)__popc(vbits);
    coded_groups += ncoded;
    const uint32_t ftarget = ncoded * 8;

    // ---- decode every coded group of the round ----
    uint32_t f = 0;
    if (n >= 8 && f < ftarget) {   // words left over from the previous round
      stage[stage_at(f, lane)] = (uint32_t)acc;
      acc >>= 32;
      n -= 8;
      ++f;
    }
    while (f < ftarget) {
      if (avail < 24) refill();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint2 e = lut[(uint32_t)(buf >> (64 - kLutBits))];
        uint32_t cnt = ((e.x >> 8) & 0xFFu) >> 2, nb = e.x & 0xFFu, syms = e.y;
        if (f >= ftarget) {   // second lookup after the round is complete: discard it
          cnt = 0;
          nb = 0;
          syms = 0;
        } else if (e.x & kLutInvalid) {   // no codeword starts here: corrupt stream (entry still advances)
          bad = true;
        }
        buf <<= nb;
        avail -= (int)nb;
        consumed += nb;
        acc |= (uint64_t)syms << (4 * n);
        n += (int)cnt;
        if (n >= 8) {
          stage[stage_at(f, lane)] = (uint32_t)acc;
          acc >>= 32;
          n -= 8;
          ++f;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // ---- cooperative copy-out of the wave's round ----
    // the wave covers 64 owners x CH groups x 64 weights; 16 weights per lane-step
    const uint32_t per_owner = CH * 64u;
    const uint32_t steps = 4u * CH;     // 64 owners * per_owner weights / 1024 weights per step
    constexpr int U = 4;
    for (uint32_t it = 0; it < steps; it += U) {
      uint4 ev[U], sv[U] = {};
      uint64_t el[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t e = (it + (uint32_t)u) * 1024u + (uint32_t)lane * 16u;
        const uint32_t L = e / per_owner, o = e % per_owner, j = o >> 6, w16 = o & 63u;
        const uint32_t fl = (uint32_t)__shfl((int)vbits, (int)L, 64);
        const uint32_t rk = (uint32_t)__shfl((int)rank0, (int)L, 64);
        const uint32_t ng = (uint32_t)__shfl((int)ngroups, (int)L, 64);
        const uint64_t sL = sbase + L;
        ok[u] = sL < a.segments && j < ng;
        el[u] = (sL * SG + (uint64_t)r * CH + j) * 64u + w16;
        const uint32_t below = fl & ((1u << j) - 1u);
        if (ok[u] && ((fl >> j) & 1u)) {
          const uint32_t rank = rk + (uint32_t)__popc(below);
          ev[u] = *reinterpret_cast<const uint4*>(vexp + (uint64_t)rank * 64u + w16);
          if (MODE == kDecodeNibble) ev[u] = make_uint4(0, 0, 0, 0);
        } else {
          const uint32_t slot = 8u * (j - (uint32_t)__popc(below)) + (w16 >> 3);
          const uint32_t n0 = stage[stage_at(slot, L)], n1 = stage[stage_at(slot + 1, L)];
          if (MODE == kDecodeNibble) {
            ev[u] = make_uint4(n0, n1, 0, 0);
          } else {
            ev[u] = pal16_any(n0, n1, pal);
          }
        }
        if (MODE == kDecodeFull && ok[u]) sv[u] = *reinterpret_cast<const uint4*>(smp + el[u]);
        if (MODE == kDecodeFp8 && ok[u]) {
          const uint2 q = *reinterpret_cast<const uint2*>(smp + el[u] / 2u);
          sv[u] = make_uint4(q.x, q.y, 0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        if (MODE == kDecodeNibble) {
          *reinterpret_cast<uint2*>((uint8_t*)a.out + el[u] / 2) = make_uint2(ev[u].x, ev[u].y);
        } else if (MODE == kDecodeExponent) {
          *reinterpret_cast<uint4*>((uint8_t*)a.out + el[u]) = ev[u];
        } else if (MODE == kDecodeFp8) {
          uint4 o;
          fp8_rebuild8(sv[u].x, ev[u].x, ev[u].y, o.x, o.y);
          fp8_rebuild8(sv[u].y, ev[u].z, ev[u].w, o.z, o.w);
          *reinterpret_cast<uint4*>((uint8_t*)a.out + el[u]) = o;
        } else {
          uint4 o0, o1;
          rebuild4(sv[u].x, ev[u].x, o0.x, o0.y);
          rebuild4(sv[u].y, ev[u].y, o0.z, o0.w);
          rebuild4(sv[u].z, ev[u].z, o1.x, o1.y);
          rebuild4(sv[u].w, ev[u].w, o1.z, o1.w);
          uint4* dst = reinterpret_cast<uint4*>((uint16_t*)a.out + el[u]);
          dst[0] = o0;
          dst[1] = o1;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // segment accounting: the codes actually used must end inside the last
  // word of the segment (segments are word aligned, pad bits follow)
  if (sval) {
    uint32_t left_bits = 0;
    for (int i = 0; i < n; ++i) left_bits += (uint32_t)((a.len_pack >> (4 * ((acc >> (4 * i)) & 15u))) & 15u);
    const uint32_t used = consumed - left_bits;
    const uint32_t words = w1 - w0;
    if (coded_groups == 0) {
      if (words != 0) bad = true;
    } else if (used > 32u * words || used <= 32u * (words - 1u)) {
      bad = true;
    }
  }
  if (bad) atomicOr(a.corrupt, 1);
}


// ---------------------------------------------------------------------------------
// Staged decoder.  Same output as k_decode_direct, but every wave first copies
// the contiguous stream range of its 64 segments into LDS with coalesced
// 16-byte loads, so the per-lane bit reader never waits on HBM; the next word
// is read from LDS one refill ahead.  Rounds are CH groups (1 or 2) and the
// global loads that the copy-out needs (sign+mantissa bytes for the BF16
// rebuild, exponents of verbatim groups) are issued before the round's decode
// loop so that the loop hides their latency.  LDS per block: the 32 KB table
// (static), then per wave a 64 x (8 CH + 1)-word stage and a wave_span-word
// stream copy (dynamic).  The host picks CH and the waves per block that keep
// the most waves resident under the 160 KB LDS of a CU.
// stage words per lane: 8 per group of the round, plus one so that the odd
// stride spreads lanes over the LDS banks
template <int CH>
constexpr uint32_t staged_stride() { return 8u * CH + 1u; }
// Largest block: sixteen waves for one-group rounds (their kernels fit the
// 128 registers a wave then gets), eight for two-group rounds.
template <int CH>
constexpr uint32_t staged_max_threads() { return CH == 1 ? 1024u : 512u; }

template <int MODE, int CH, bool RUN, bool NT>
__global__ __launch_bounds__(staged_max_threads<CH>()) void k_decode_staged(DecodeArgs a) {
  constexpr uint32_t kStagedStride = staged_stride<CH>();
  constexpr uint32_t kStagedStage = 64 * kStagedStride;
  __shared__ __attribute__((aligned(16))) uint2 lut[1 << kLutBits];
  extern __shared__ uint32_t dyn[];
  const int lane = threadIdx.x & 63, wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t span = (a.wave_span + 8u + 3u) & ~3u;   // + read slack, 16-byte multiple
  uint32_t* stage = dyn + (uint32_t)wave * (kStagedStage + span);
  uint32_t* sbuf = stage + kStagedStage;

  const uint64_t sbase = (uint64_t)blockIdx.x * blockDim.x + (uint64_t)wave * 64;
  const uint64_t s = sbase + (uint64_t)lane;
  const bool sval = s < a.segments;
  const bool wval = sbase < a.segments;
  const uint32_t SG = a.seg_groups;
  const uint32_t rounds = SG / CH;
  const uint32_t w0 = sval ? a.seg_off[s] : 0u;
  const uint32_t w1 = sval ? a.seg_off[s + 1] : 0u;
  const uint32_t ws0 = wval ? (a.seg_off[sbase] & ~3u) : 0u;
  const uint32_t we1 = wval ? a.seg_off[sbase + 64 < a.segments ? sbase + 64 : a.segments] : 0u;

  // verbatim flags of the whole segment (<= 64 groups, SG-aligned) and the
  // rank of its first group
  uint64_t segbits = 0;
  uint32_t rank_seg = 0;
  uint32_t seg_ng = 0;
  if (sval) {
    const uint64_t g0 = s * SG;
    const uint64_t left = a.groups - g0;
    seg_ng = left < SG ? (uint32_t)left : SG;
    const uint32_t sh = (uint32_t)(g0 & 31);
    const uint32_t fw = a.vflags[g0 >> 5];
    uint64_t bits = fw >> sh;
    if (SG == 64 && seg_ng > 32) bits |= (uint64_t)a.vflags[(g0 >> 5) + 1] << 32;
    segbits = seg_ng == 64 ? bits : (bits & ((1ull << seg_ng) - 1ull));
    rank_seg = a.vrank[g0 >> 5] + (uint32_t)__popc(fw & ((1u << sh) - 1u));
  }

  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.stream, (short)0, (int)(a.stream_words * 4u), 0x00020000);
  // The copy-out's verbatim-exponent loads and all its stores go through
  // buffer resources, lanes with nothing to move giving an offset past the
  // end: no branches, so every path issues the same memory operations and
  // the waits at the head of the next round count only the loads they need
  // (behind branches they drained the previous round's stores).  The output
  // resource starts at the wave's first weight; the host keeps the verbatim
  // section under kRecordsMax.
  const uint64_t wel0 = wval ? sbase * SG * 64u : 0u;
  const uint64_t ob0 = out_bytes<MODE>(wel0), oend = out_bytes<MODE>(a.groups * 64u);
  const uint64_t oleft = oend > ob0 ? oend - ob0 : 0u;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (uint8_t*)a.out + ob0, (short)0, (int)(oleft < kRecordsMax ? oleft : kRecordsMax), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.vexp, (short)0, (int)(a.vexp_bytes < kRecordsMax ? a.vexp_bytes : kRecordsMax), 0x00020000);
  // stream range of this wave -> LDS (16 bytes per lane per load) and the
  // block's share of the table: every load of a batch is issued before the
  // first LDS write waits on them, so the copy costs one memory latency per
  // batch rather than one per 16-byte piece.  Pieces past the range load
  // from past the resource's end (zero) and are not written.
  const uint32_t nwords = we1 - ws0;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)a.lut, (short)0, (int)kLutBytes, 0x00020000);
  constexpr uint32_t kCopyBatch = 8;   // 2048 stream words per wave per batch
  constexpr uint32_t kLutBatch = 4;    // table pieces per thread per batch
  constexpr uint32_t kLutPieces = kLutBytes / 16u;
  const uint32_t nthreads = blockDim.x;
  for (uint32_t base = 0, lbase = 0; base < nwords || lbase < kLutPieces;
       base += 256u * kCopyBatch, lbase += kLutBatch * nthreads) {
    uint4 v[kCopyBatch], t[kLutBatch];
#pragma unroll
    for (uint32_t j = 0; j < kCopyBatch; ++j) {
      const uint32_t i = base + j * 256u + (uint32_t)lane * 4u;
      v[j] = load_chunk<MODE == kDecodeNibble>(rs, i < nwords ? ws0 + i : kPastEnd / 4u);
    }
#pragma unroll
    for (uint32_t j = 0; j < kLutBatch; ++j) {
      const uint32_t i = lbase + j * nthreads + threadIdx.x;
      t[j] = buf_load16(rl, i < kLutPieces ? i * 16u : kPastEnd);
    }
#pragma unroll
    for (uint32_t j = 0; j < kLutBatch; ++j) {
      const uint32_t i = lbase + j * nthreads + threadIdx.x;
      if (i < kLutPieces) reinterpret_cast<uint4*>(lut)[i] = t[j];
    }
#pragma unroll
    for (uint32_t j = 0; j < kCopyBatch; ++j) {
      const uint32_t i = base + j * 256u + (uint32_t)lane * 4u;
      if (i < nwords) *reinterpret_cast<uint4*>(&sbuf[i]) = v[j];
    }
  }
  __syncthreads();
  if (!wval) return;

  const uint32_t p0 = sval ? w0 - ws0 : 0u;
  uint32_t p = p0;   // next LDS word to shift into the buffer
  uint64_t buf = ((uint64_t)sbuf[p] << 32) | (uint64_t)sbuf[p + 1];
  p += 2;
  uint32_t nw = sbuf[p];
  int avail = 64;
  uint32_t flags = 0;     // OR of the first words of all table entries used
  uint64_t acc = 0;
  uint32_t sh4 = 0;       // 4 x pending nibbles in acc
  // Takes the next word when fewer than 24 bits are buffered (enough for two
  // lookups).  Selects instead of a branch: the lanes of a wave need words at
  // different times, and a branch would run the refill under an exec mask
  // almost every time anyway.
  auto refill = [&]() {
    const bool need = avail < 24;
    buf |= (uint64_t)(need ? nw : 0u) << ((uint32_t)(32 - avail) & 63u);
    avail += need ? 32 : 0;
    p += need ? 1u : 0u;
    nw = sbuf[min(p, span - 1u)];   // a corrupt stream cannot read past the copy
  };
  uint32_t coded_groups = 0;
  const PalView pal = a.pal;
  const uint8_t* __restrict__ smp = a.sm;
  constexpr uint32_t per_owner = CH * 64u;
  constexpr int STEPS = 4 * CH;   // 64 owners * per_owner weights / 1024 per step

  // Full decode with one-group rounds: an owner's sign+mantissa bytes of
  // rounds 2i and 2i+1 are the two halves of one 128-byte line, so both are
  // loaded in round 2i (the second half waits in svn) and each line is read
  // once instead of twice.
  // Exponent decode likewise writes an owner's rounds 2i and 2i+1 together:
  // round 2i's 16-byte pieces wait in exn and are stored beside round 2i+1's,
  // so every 128-byte line of output is written whole.
  uint4 svn[STEPS], exn[STEPS];
  uint32_t deferred = 0;   // bit u: exn[u] holds a piece of the previous round
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    svn[u] = make_uint4(0, 0, 0, 0);
    exn[u] = make_uint4(0, 0, 0, 0);
  }
  // Transcode with one-group rounds: a group's slots are a quarter of a
  // 128-byte line whose other quarters come in the owner's next rounds.
  // Stored round by round, L2 sometimes wrote the line back between rounds
  // (twice the bytes, depending on how blocks fell on the XCDs).  When
  // segments are whole lines (groups per segment a multiple of 4) the quarter
  // is the round mod 4 for every owner, so each step keeps its quarters in
  // fixed registers and stores the four back to back in the line's last
  // round (or the segment's last, for a short final segment).
  constexpr int HOLD = MODE == kDecodeNibble && CH == 1 ? 3 : 1;
  const bool whole_lines = (SG & 3u) == 0;
  uint2 held[STEPS][HOLD];
#pragma unroll
  for (int u = 0; u < STEPS; ++u)
#pragma unroll
    for (int h = 0; h < HOLD; ++h) held[u][h] = make_uint2(0, 0);

  // Copy-out step u of a lane serves the same owner lane in every round, so
  // the owner's verbatim flags, first rank and group count are fetched once
  // here; each round then finds its flags and ranks without cross-lane
  // shuffles.  Owners past the last segment have no groups.
  uint32_t obl[STEPS], obh[STEPS], ork[STEPS], ong[STEPS];
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const int L = (int)(((uint32_t)u * 1024u + (uint32_t)lane * 16u) / per_owner);
    obl[u] = (uint32_t)__shfl((int)(uint32_t)segbits, L, 64);
    obh[u] = (uint32_t)__shfl((int)(uint32_t)(segbits >> 32), L, 64);
    ork[u] = (uint32_t)__shfl((int)rank_seg, L, 64);
    ong[u] = (uint32_t)__shfl((int)seg_ng, L, 64);
  }

  for (uint32_t r = 0; r < rounds; ++r) {
    const uint32_t ng = seg_ng > r * CH ? (seg_ng - r * CH < CH ? seg_ng - r * CH : CH) : 0u;
    const bool pair_first = MODE == kDecodeFull && CH == 1 && (r & 1u) == 0;
    const bool pair_second = MODE == kDecodeFull && CH == 1 && (r & 1u) == 1;
    // one output byte per weight (exponents, FP8): an owner's two groups of a
    // 128-byte line are stored together in the odd round
    const bool defer_first = (MODE == kDecodeExponent || MODE == kDecodeFp8) && CH == 1 && (r & 1u) == 0;
    uint32_t has_next = 0;   // bit u: this step's owner has a group in round r+1
    const uint32_t vbits = (uint32_t)(segbits >> (r * CH)) & ((1u << CH) - 1u) & ((1u << ng) - 1u);
    const uint32_t ncoded = ng - (uint32_t)__popc(vbits);
    coded_groups += ncoded;
    const uint32_t ftarget = ncoded * 8;

    // ---- issue the copy-out loads of this round ----
    uint4 ev[STEPS], sv[STEPS];
    uint64_t el[STEPS];
    uint32_t info[STEPS];   // bit 31: ok, bit 30: verbatim, low bits: stage slot | owner << 8
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const uint32_t e = (uint32_t)u * 1024u + (uint32_t)lane * 16u;
      const uint32_t L = e / per_owner, o = e % per_owner, j = o >> 6, w16 = o & 63u;
      const uint32_t gi = r * CH + j;   // group index in the owner's segment
      const uint64_t ob = ((uint64_t)obh[u] << 32) | obl[u];
      const bool ok = gi < ong[u];
      const bool verb = ok && ((ob >> gi) & 1u);
      const uint32_t below = (uint32_t)(ob >> (r * CH)) & ((1u << j) - 1u);   // the round's verbatim groups before j
      const uint64_t sL = sbase + L;
      el[u] = (sL * SG + gi) * 64u + w16;
      info[u] = (ok ? 0x80000000u : 0u) | (verb ? 0x40000000u : 0u) | (L << 8) |
                (8u * (j - (uint32_t)__popc(below)) + (w16 >> 3));
      ev[u] = make_uint4(0, 0, 0, 0);
      sv[u] = make_uint4(0, 0, 0, 0);
      if constexpr (MODE != kDecodeNibble) {
        const uint32_t rank = ork[u] + (uint32_t)__popcll(ob & ((1ull << gi) - 1ull));
        ev[u] = buf_load16(rv, verb ? rank * 64u + w16 : kPastEnd);
      }
      // sign+mantissa loads read index 0 for steps that store nothing
      if (pair_second) {
        sv[u] = svn[u];
      } else if (MODE == kDecodeFull) {
        sv[u] = *reinterpret_cast<const uint4*>(smp + (ok ? el[u] : 0u));
      } else if (MODE == kDecodeFp8) {   // 16 packed sign+mantissa nibbles
        const uint2 q = *reinterpret_cast<const uint2*>(smp + (ok ? el[u] / 2u : 0u));
        sv[u] = make_uint4(q.x, q.y, 0u, 0u);
      }
      const bool next = (r + 1) * CH < ong[u];   // the owner has a group in round r+1 (CH == 1)
      if (defer_first) has_next |= next ? (1u << u) : 0u;
      if (pair_first) svn[u] = *reinterpret_cast<const uint4*>(smp + (next ? el[u] + 64u : 0u));
    }

    // ---- decode every coded group of the round (LDS only) ----
    // One lookup: the entry's slots join the nibble accumulator and its low
    // word is written to the lane's current stage word; once 32 bits are
    // pending the write was the complete word and the pointer moves on.
    // Straight-line, so lanes never wait on each other's branches.
    uint32_t* wp = stage + (uint32_t)lane * kStagedStride;
    uint32_t* const wend = wp + ftarget;
    uint32_t* const wlast = wend - 1;
    auto lookup = [&]() {
      const uint2 e = lut[(uint32_t)(buf >> (64 - kLutBits))];
      flags |= e.x;
      buf <<= (e.x & 63u);
      avail -= (int)(e.x & 0xFFu);
      acc |= (uint64_t)e.y << sh4;
      sh4 += (e.x >> 8) & 0xFFu;
      *wp = (uint32_t)acc;
      const uint32_t full = sh4 & 32u;
      acc >>= full;
      sh4 -= full;
      wp += full >> 5;
    };
    // two lookups per refill while at least two stage words remain (each
    // lookup completes at most one word), then single lookups
    while (wp < wlast) {
      refill();
      lookup();
      lookup();
    }
    while (wp < wend) {
      refill();
      lookup();
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();

    // ---- copy-out ----
    // straight-line data path (the stage words are read for every step: the
    // slot stays inside the owner's stage row); only the stores are predicated
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const bool ok = (info[u] >> 31) & 1u, verb = (info[u] >> 30) & 1u;
      const uint32_t L = (info[u] >> 8) & 63u, slot = info[u] & 0xFFu;
      const uint32_t n0 = stage[L * kStagedStride + slot], n1 = stage[L * kStagedStride + slot + 1];
      uint4 ex;
      if constexpr (MODE == kDecodeNibble) {
        ex = make_uint4(verb ? 0u : n0, verb ? 0u : n1, 0u, 0u);   // verbatim groups: slot 0
      } else {
        const uint4 pe = pal16<RUN>(n0, n1, pal);
        ex.x = verb ? ev[u].x : pe.x;
        ex.y = verb ? ev[u].y : pe.y;
        ex.z = verb ? ev[u].z : pe.z;
        ex.w = verb ? ev[u].w : pe.w;
      }
      const uint32_t rel = (uint32_t)(el[u] - wel0);   // weights past the wave's first (when ok)
      if constexpr (MODE == kDecodeNibble && CH == 1) {
        if (whole_lines) {
          const uint32_t q = r & 3u;   // the group's quarter of its line, the same for every owner
          // no loads in this mode's rounds, so branching around stores costs no waits
          if (ok && (q == 3u || r + 1u >= ong[u])) {
            const uint32_t b = rel / 2u;   // quarter i of the line sits at b - 32 (q - i)
            buf_store8(ro, q >= 1u ? b - 32u * q : kPastEnd, held[u][0].x, held[u][0].y);
            buf_store8(ro, q >= 2u ? b - 32u * (q - 1u) : kPastEnd, held[u][1].x, held[u][1].y);
            buf_store8(ro, q >= 3u ? b - 32u : kPastEnd, held[u][2].x, held[u][2].y);
            buf_store8(ro, b, ex.x, ex.y);
          }
          // fixed registers: q is uniform, so these are scalar-conditioned moves
          if (q == 0u) held[u][0] = make_uint2(ex.x, ex.y);
          if (q == 1u) held[u][1] = make_uint2(ex.x, ex.y);
          if (q == 2u) held[u][2] = make_uint2(ex.x, ex.y);
        } else {
          buf_store8(ro, ok ? rel / 2u : kPastEnd, ex.x, ex.y);
        }
      } else if constexpr (MODE == kDecodeNibble) {
        buf_store8(ro, ok ? rel / 2u : kPastEnd, ex.x, ex.y);
      } else if constexpr (MODE == kDecodeExponent || MODE == kDecodeFp8) {
        uint4 ob = ex;
        if constexpr (MODE == kDecodeFp8) {
          fp8_rebuild8(sv[u].x, ex.x, ex.y, ob.x, ob.y);
          fp8_rebuild8(sv[u].y, ex.z, ex.w, ob.z, ob.w);
        }
        if constexpr (CH == 1)   // the other half of this line, from the previous round
          buf_store16<NT>(ro, ((deferred >> u) & 1u) ? rel - 64u : kPastEnd, exn[u]);
        const bool hold = defer_first && ((has_next >> u) & 1u);
        buf_store16<NT>(ro, ok && !hold ? rel : kPastEnd, ob);
        exn[u] = ob;   // used next round only when held
      } else {
        uint4 o0, o1;
        rebuild4(sv[u].x, ex.x, o0.x, o0.y);
        rebuild4(sv[u].y, ex.y, o0.z, o0.w);
        rebuild4(sv[u].z, ex.z, o1.x, o1.y);
        rebuild4(sv[u].w, ex.w, o1.z, o1.w);
        const uint32_t off = ok ? rel * 2u : kPastEnd;
        buf_store16<NT>(ro, off, o0);
        buf_store16<NT>(ro, off + 16u, o1);
      }
    }
    deferred = defer_first ? has_next : 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  bool bad = (flags & kLutInvalid) != 0;
  if (sval) {
    uint32_t left_bits = 0;
    for (uint32_t i = 0; i < sh4 / 4u; ++i)
      left_bits += (uint32_t)((a.len_pack >> (4 * ((acc >> (4 * i)) & 15u))) & 15u);
    const uint32_t words_in = p - p0;
    const uint32_t used = 32u * words_in - (uint32_t)avail - left_bits;
    const uint32_t words = w1 - w0;
    if (coded_groups == 0) {
      if (words != 0) bad = true;
    } else if (used > 32u * words || used <= 32u * (words - 1u)) {
      bad = true;
    }
  }
  if (bad) atomicOr(a.corrupt, 1);
}

constexpr uint32_t kMaxLds = 160u * 1024u;                      // per workgroup on gfx950
constexpr uint32_t kMaxDynLds = kMaxLds - kLutBytes;  // the table is static

// dynamic LDS of the staged kernel per wave (the table is static)
template <int CH>
uint32_t staged_wave_bytes(const DecodeArgs& a) {
  return 4u * (64u * staged_stride<CH>() + ((a.wave_span + 8u + 3u) & ~3u));
}

// Waves per block.  Every block copies the table, so on a small grid larger
// blocks leave CUs idle and on a large one smaller blocks spend LDS on copies
// of the table that could hold more waves.  The choice minimises the most
// waves any CU runs over the launch (blocks are dealt to CUs in turn), then
// maximises the waves a CU holds at once (LDS permitting; at most 16, and 8
// for two-group rounds, whose full-decode kernel takes about 200 registers),
// then takes the smaller block.  0 waves if one wave does not fit.
struct StagedShape {
  uint32_t wpb = 0;        // waves per block
  uint64_t load = 0;       // most waves one CU runs
  uint32_t resident = 0;   // waves a CU holds at once
};

template <int CH>
StagedShape staged_shape(const DecodeArgs& a) {
  const uint32_t per_wave = staged_wave_bytes<CH>(a);
  const uint64_t waves = (a.segments + 63u) / 64u;
  const uint64_t cus = (uint64_t)device_cus();
  StagedShape best;
  for (uint32_t wpb = 1; wpb <= staged_max_threads<CH>() / 64u; ++wpb) {
    const uint32_t dyn = wpb * per_wave;
    if (dyn > kMaxDynLds) break;
    uint32_t per_cu = kMaxLds / (dyn + kLutBytes);   // blocks a CU holds at once
    constexpr uint32_t cap = CH == 1 ? 16u : 8u;
    if (per_cu * wpb > cap) per_cu = cap / wpb;
    if (per_cu == 0) break;
    const uint64_t blocks = (waves + wpb - 1) / wpb;
    const uint64_t rounds = (blocks + cus - 1) / cus;   // blocks dealt to the busiest CU
    const uint64_t load = rounds * wpb;
    const uint32_t resident = (uint32_t)((rounds < per_cu ? rounds : per_cu) * wpb);
    if (best.wpb == 0 || load < best.load || (load == best.load && resident > best.resident)) {
      best.wpb = wpb;
      best.load = load;
      best.resident = resident;
    }
  }
  return best;
}

template <int MODE, int CH, bool RUN, bool NT>
hipError_t launch_staged_pal(const DecodeArgs& a, uint32_t wpb, hipStream_t s) {
  hipError_t e = allow_dynamic_lds((const void*)k_decode_staged<MODE, CH, RUN, NT>, (int)kMaxDynLds);
  if (e != hipSuccess) return e;
  const uint64_t threads = 64ull * wpb;
  const uint64_t blocks = (a.segments + threads - 1) / threads;
  hipLaunchKernelGGL((k_decode_staged<MODE, CH, RUN, NT>), dim3((uint32_t)blocks), dim3((uint32_t)threads),
                     wpb * staged_wave_bytes<CH>(a), s, a);
  return hipGetLastError();
}

// the palette kind is a template parameter (a run of exponents is a bytewise
// add); the transcode never looks the palette up.  Store policy: see
// buf_store16.
template <int MODE, int CH>
hipError_t launch_staged(const DecodeArgs& a, uint32_t wpb, hipStream_t s) {
  if constexpr (MODE == kDecodeNibble) {
    return launch_staged_pal<MODE, CH, false, false>(a, wpb, s);
  } else if constexpr (MODE == kDecodeExponent) {
    return a.pal.run ? launch_staged_pal<MODE, CH, true, true>(a, wpb, s)
                     : launch_staged_pal<MODE, CH, false, true>(a, wpb, s);
  } else {
    const bool nt = a.groups * 64u * (MODE == kDecodeFp8 ? 1u : 2u) > kCachedOutputMax;
    if (a.pal.run)
      return nt ? launch_staged_pal<MODE, CH, true, true>(a, wpb, s) : launch_staged_pal<MODE, CH, true, false>(a, wpb, s);
    return nt ? launch_staged_pal<MODE, CH, false, true>(a, wpb, s) : launch_staged_pal<MODE, CH, false, false>(a, wpb, s);
  }
}

template <int MODE>
hipError_t launch_mode(const DecodeArgs& a, uint32_t blocks, hipStream_t s) {
  const char* force = std::getenv("UW_DECODE_DIRECT");   // selects the fallback kernel (tests)
  if (a.wave_span > 0 && a.vexp_bytes <= kRecordsMax && !(force && force[0] == '1')) {
    // rounds of two groups where that spreads the waves as well as rounds of one
    const StagedShape s1 = staged_shape<1>(a);
    const StagedShape s2 = a.seg_groups >= 2 ? staged_shape<2>(a) : StagedShape{};
    if (s2.wpb > 0 && (s1.wpb == 0 || (s2.load <= s1.load && s2.resident >= s1.resident)))
      return launch_staged<MODE, 2>(a, s2.wpb, s);
    if (s1.wpb > 0) return launch_staged<MODE, 1>(a, s1.wpb, s);
  }
  hipLaunchKernelGGL(k_decode_direct<MODE>, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int mode, hipStream_t s) {
  const uint64_t blocks = (a.segments + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
  switch (mode) {
    case kDecodeNibble: return launch_mode<kDecodeNibble>(a, (uint32_t)blocks, s);
    case kDecodeExponent: return launch_mode<kDecodeExponent>(a, (uint32_t)blocks, s);
    case kDecodeFp8: return launch_mode<kDecodeFp8>(a, (uint32_t)blocks, s);
    default: return launch_mode<kDecodeFull>(a, (uint32_t)blocks, s);
  }
}

}  // namespace uw
