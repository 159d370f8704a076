// uwo.cpp -- CPU oracle for the Unweight-style lossless BF16 exponent codec.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
// includes this file; only the test-suite, the smoke check and the CPU-baseline
// leg of the benchmark load it (through oracle/oracle.py).  It shares no code,
// header, table or constant generator with the HIP library: every step below is
// written out plainly, one element or one bit at a time, so that a reader can
// check it against the method's description by eye.
//
// Sources (cited by page title and section heading):
//   [EVC]  "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
//          (easyvibecoding.app/curated/736).
//   [GT]   goodtech.info, "Cloudflare Unweight" article, section
//          "La magie du code de Huffman".
//   [RFC1951] DEFLATE, section 3.2.2 (canonical Huffman code assignment).
//   [LH90] Larmore & Hirschberg, "A fast algorithm for optimal length-limited
//          Huffman codes", JACM 1990 (package-merge).
//   [SP]   saidapartage.blog, "Cloudflare Unweight : -22 % sur le poids de vos
//          LLM, sans perdre un bit", section "Un complément, pas un remplaçant".
//   [OFP8] OCP 8-bit Floating Point Specification (OFP8), the E4M3 format.
//
// What the pages fix and what is a reading (the UWF1 encoding):
//   * BF16 = 1 sign bit, 8 exponent bits, 7 mantissa bits; sign and mantissa
//     are kept as they are, only the exponent byte is entropy-coded
//     ([EVC] "BF16權重壓縮原理"; [GT] "La magie du code de Huffman").
//   * A few exponent values dominate; the 16 most frequent form a palette and
//     a 4-bit index addresses it ([EVC] "BF16權重壓縮原理", "四種執行管道").
//   * A row of 64 weights holding any exponent outside that palette is kept
//     verbatim, decided once per row ([EVC] "BF16權重壓縮原理").
//   * Everything else (byte packing of sign+mantissa, the length limit of the
//     code, tie-breaks, bit order, segmenting) is the UWF1 reading documented
//     alongside the library; this file is the executable statement of it.
//
// Already-quantised weights ([SP]; [GT] section "Open source"): the pages say
// the coding also applies on top of quantisation and give no more.  The
// reading here (UWF8) is the plainest one for FP8 E4M3 weights: the 4-bit
// exponent field is the coded symbol, exactly as the BF16 exponent byte is,
// and sign plus mantissa are kept as a 4-bit nibble.  E4M3 has at most 16
// exponent values, so the palette always holds them all and no group is ever
// verbatim.
//
// Parity pins for each function live in tests/test_oracle_*.py.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

namespace {

constexpr int kLMax = 12;         // longest allowed code length (UWF1 reading)
constexpr int kGroup = 64;        // weights per verbatim decision ([EVC] "BF16權重壓縮原理")
constexpr int kPalette = 16;      // palette size ([EVC] "BF16權重壓縮原理")

enum {
  UWO_OK = 0,
  UWO_ERR_INVALID = -1,
  UWO_ERR_UNSUPPORTED = -2,
  UWO_ERR_NOMEM = -3,
  UWO_ERR_CORRUPT = -5,
};

struct Oracle {
  // shape
  uint64_t rows = 0, cols = 0, numel = 0, groups = 0, segments = 0, flag_words = 0;
  uint32_t seg_groups = 0, layout = 0;
  // tables
  uint64_t hist[256] = {};
  uint32_t palette_size = 0;
  uint8_t palette[kPalette] = {};   // ascending, unused entries 0
  int slot_of[256];                 // -1 when the exponent is not in the palette
  uint64_t coded_count[kPalette] = {};
  uint32_t n_coded = 0;
  uint8_t code_len[kPalette] = {};
  uint16_t code[kPalette] = {};
  // counts
  uint64_t verbatim_groups = 0;     // V
  uint64_t stream_words = 0;        // W (without the two slack words)
  uint64_t code_bits = 0;           // sum over segments of the bits written
  // sections
  std::vector<uint8_t> sm;          // sign+mantissa byte of every element
  std::vector<uint32_t> vflags;     // bit t of word w = group 32w+t is verbatim
  std::vector<uint32_t> vrank;      // verbatim groups before word w
  std::vector<uint8_t> vexp;        // 64 raw exponents per verbatim group
  std::vector<uint32_t> seg_off;    // word offset of each segment, S+1 entries
  std::vector<uint32_t> stream;     // W + 2 words, MSB-first codes
  bool fp8 = false;                 // UWF8: sm holds packed sign+mantissa nibbles
};

// ---- field split and rebuild ([EVC] "BF16權重壓縮原理") ----------------------
// sign = bit 15, exponent = bits 14..7, mantissa = bits 6..0.
// UWF1 reading: the kept byte is (sign << 7) | mantissa.
inline uint8_t exponent_of(uint16_t b) { return (uint8_t)((b >> 7) & 0xFF); }
inline uint8_t sign_mantissa_of(uint16_t b) {
  uint8_t sign = (uint8_t)((b >> 15) & 1);
  uint8_t mant = (uint8_t)(b & 0x7F);
  return (uint8_t)((sign << 7) | mant);
}
inline uint16_t rebuild(uint8_t sm, uint8_t e) {
  uint16_t sign = (uint16_t)((sm >> 7) & 1);
  uint16_t mant = (uint16_t)(sm & 0x7F);
  return (uint16_t)((sign << 15) | ((uint16_t)e << 7) | mant);
}

// ---- FP8 E4M3 field split and rebuild ([OFP8]; UWF8 reading) ---------------
// sign = bit 7, exponent = bits 6..3, mantissa = bits 2..0.
// UWF8 reading: the kept nibble is (sign << 3) | mantissa, two per byte, the
// element with the even index in the low nibble.
inline uint8_t fp8_exponent_of(uint8_t b) { return (uint8_t)((b >> 3) & 0xF); }
inline uint8_t fp8_sign_mantissa_of(uint8_t b) {
  uint8_t sign = (uint8_t)((b >> 7) & 1);
  uint8_t mant = (uint8_t)(b & 0x7);
  return (uint8_t)((sign << 3) | mant);
}
inline uint8_t fp8_rebuild(uint8_t smn, uint8_t e) {
  uint8_t sign = (uint8_t)((smn >> 3) & 1);
  uint8_t mant = (uint8_t)(smn & 0x7);
  return (uint8_t)((sign << 7) | ((e & 0xF) << 3) | mant);
}

// ---- package-merge ([LH90]) --------------------------------------------------
// Optimal prefix-code lengths, none longer than lmax, for n >= 2 positive
// weights.  Items are (weight, list of symbols); leaves are ordered by
// (weight, symbol index) ascending and, when a leaf and a package weigh the
// same, the leaf goes first.
struct PMItem {
  uint64_t weight;
  std::vector<int> symbols;
};

bool package_merge(const uint64_t* weight, int n, int lmax, uint8_t* len_out) {
  if (n < 2 || n > (1 << lmax)) return false;
  std::vector<PMItem> leaves;
  for (int i = 0; i < n; ++i) leaves.push_back(PMItem{weight[i], {i}});
  std::stable_sort(leaves.begin(), leaves.end(), [](const PMItem& a, const PMItem& b) {
    if (a.weight != b.weight) return a.weight < b.weight;
    return a.symbols[0] < b.symbols[0];
  });
  std::vector<PMItem> list = leaves;
  for (int round = 0; round < lmax - 1; ++round) {
    // package adjacent pairs of the current list
    std::vector<PMItem> packages;
    for (size_t i = 0; i + 1 < list.size(); i += 2) {
      PMItem p;
      p.weight = list[i].weight + list[i + 1].weight;
      p.symbols = list[i].symbols;
      p.symbols.insert(p.symbols.end(), list[i + 1].symbols.begin(), list[i + 1].symbols.end());
      packages.push_back(p);
    }
    // merge with the leaves; on equal weight the leaf comes first
    std::vector<PMItem> merged;
    size_t a = 0, b = 0;
    while (a < leaves.size() || b < packages.size()) {
      bool take_leaf;
      if (a >= leaves.size()) take_leaf = false;
      else if (b >= packages.size()) take_leaf = true;
      else take_leaf = leaves[a].weight <= packages[b].weight;
      merged.push_back(take_leaf ? leaves[a++] : packages[b++]);
    }
    list = merged;
  }
  for (int i = 0; i < n; ++i) len_out[i] = 0;
  for (int i = 0; i < 2 * n - 2; ++i)
    for (int s : list[(size_t)i].symbols) len_out[s]++;
  return true;
}

// ---- canonical code assignment ([RFC1951] 3.2.2) ------------------------------
void canonical_codes(const uint8_t* len, int n, uint16_t* code_out) {
  int bl_count[kLMax + 2] = {0};
  for (int i = 0; i < n; ++i)
    if (len[i] > 0) bl_count[len[i]]++;
  int next_code[kLMax + 2] = {0};
  int c = 0;
  bl_count[0] = 0;
  for (int bits = 1; bits <= kLMax; ++bits) {
    c = (c + bl_count[bits - 1]) << 1;
    next_code[bits] = c;
  }
  for (int i = 0; i < n; ++i) {
    code_out[i] = 0;
    if (len[i] > 0) code_out[i] = (uint16_t)next_code[len[i]]++;
  }
}

// ---- bit writer: MSB-first inside little-endian 32-bit words -----------------
struct BitWriter {
  std::vector<uint32_t>* words;
  uint64_t base_word;   // first word of the segment
  uint64_t bitpos = 0;  // bits written in this segment
  void put(uint32_t value, int nbits) {
    for (int i = nbits - 1; i >= 0; --i) {
      uint32_t bit = (value >> i) & 1u;
      uint64_t w = base_word + bitpos / 32;
      int shift = 31 - (int)(bitpos % 32);
      (*words)[w] |= bit << shift;
      ++bitpos;
    }
  }
};

inline bool group_is_verbatim(const Oracle& o, uint64_t g) {
  return (o.vflags[g / 32] >> (g % 32)) & 1u;
}

inline uint64_t verbatim_rank(const Oracle& o, uint64_t g) {
  // verbatim groups strictly before g
  uint32_t word = o.vflags[g / 32];
  uint32_t below = (g % 32) == 0 ? 0u : (word & ((1u << (g % 32)) - 1u));
  return o.vrank[g / 32] + (uint64_t)__builtin_popcount(below);
}

int compress(const uint16_t* w, uint64_t rows, uint64_t cols, uint32_t seg_groups,
             uint32_t layout, Oracle& o) {
  if (w == nullptr || rows == 0 || cols == 0) return UWO_ERR_INVALID;
  if (cols % kGroup != 0) return UWO_ERR_UNSUPPORTED;
  if (seg_groups == 0 || seg_groups > 64 || (seg_groups & (seg_groups - 1)) != 0)
    return UWO_ERR_INVALID;
  if (layout > 1) return UWO_ERR_INVALID;
  o.rows = rows;
  o.cols = cols;
  o.numel = rows * cols;
  o.groups = o.numel / kGroup;
  o.seg_groups = seg_groups;
  o.layout = layout;
  o.segments = (o.groups + seg_groups - 1) / seg_groups;
  o.flag_words = (o.groups + 31) / 32;

  // split; sign+mantissa section holds every element
  o.sm.resize(o.numel);
  for (uint64_t i = 0; i < o.numel; ++i) o.sm[i] = sign_mantissa_of(w[i]);

  // exponent histogram
  for (int v = 0; v < 256; ++v) o.hist[v] = 0;
  for (uint64_t i = 0; i < o.numel; ++i) o.hist[exponent_of(w[i])]++;

  // palette: the 16 most frequent exponents, ties to the smaller value,
  // stored in ascending order
  std::vector<int> candidates;
  for (int v = 0; v < 256; ++v)
    if (o.hist[v] > 0) candidates.push_back(v);
  std::sort(candidates.begin(), candidates.end(), [&](int a, int b) {
    if (o.hist[a] != o.hist[b]) return o.hist[a] > o.hist[b];
    return a < b;
  });
  size_t keep = std::min<size_t>(kPalette, candidates.size());
  std::vector<int> chosen(candidates.begin(), candidates.begin() + (long)keep);
  std::sort(chosen.begin(), chosen.end());
  o.palette_size = (uint32_t)keep;
  for (int i = 0; i < kPalette; ++i) o.palette[i] = 0;
  for (int v = 0; v < 256; ++v) o.slot_of[v] = -1;
  for (size_t i = 0; i < keep; ++i) {
    o.palette[i] = (uint8_t)chosen[i];
    o.slot_of[chosen[i]] = (int)i;
  }

  // verbatim flags and ranks
  o.vflags.assign(o.flag_words, 0u);
  o.vrank.assign(o.flag_words, 0u);
  o.verbatim_groups = 0;
  for (uint64_t g = 0; g < o.groups; ++g) {
    bool verbatim = false;
    for (int j = 0; j < kGroup; ++j)
      if (o.slot_of[exponent_of(w[g * kGroup + j])] < 0) verbatim = true;
    if (verbatim) {
      o.vflags[g / 32] |= 1u << (g % 32);
      o.verbatim_groups++;
    }
  }
  uint64_t running = 0;
  for (uint64_t wd = 0; wd < o.flag_words; ++wd) {
    o.vrank[wd] = (uint32_t)running;
    running += (uint64_t)__builtin_popcount(o.vflags[wd]);
  }

  // coded histogram: palette slots over the non-verbatim groups only
  for (int s = 0; s < kPalette; ++s) o.coded_count[s] = 0;
  for (uint64_t g = 0; g < o.groups; ++g) {
    if (group_is_verbatim(o, g)) continue;
    for (int j = 0; j < kGroup; ++j) o.coded_count[o.slot_of[exponent_of(w[g * kGroup + j])]]++;
  }

  // code lengths
  std::vector<int> active;
  for (int s = 0; s < kPalette; ++s)
    if (o.coded_count[s] > 0) active.push_back(s);
  o.n_coded = (uint32_t)active.size();
  for (int s = 0; s < kPalette; ++s) o.code_len[s] = 0;
  if (active.size() == 1) {
    o.code_len[active[0]] = 1;
  } else if (active.size() >= 2) {
    std::vector<uint64_t> wts;
    for (int s : active) wts.push_back(o.coded_count[s]);
    std::vector<uint8_t> lens(active.size());
    package_merge(wts.data(), (int)active.size(), kLMax, lens.data());
    for (size_t i = 0; i < active.size(); ++i) o.code_len[active[i]] = lens[i];
  }
  canonical_codes(o.code_len, kPalette, o.code);

  // segmented bitstream: first the bit count of every segment, then the words
  std::vector<uint64_t> seg_bits(o.segments, 0);
  for (uint64_t s = 0; s < o.segments; ++s) {
    uint64_t g_end = std::min<uint64_t>((s + 1) * seg_groups, o.groups);
    for (uint64_t g = s * seg_groups; g < g_end; ++g) {
      if (group_is_verbatim(o, g)) continue;
      for (int j = 0; j < kGroup; ++j)
        seg_bits[s] += o.code_len[o.slot_of[exponent_of(w[g * kGroup + j])]];
    }
  }
  o.seg_off.assign(o.segments + 1, 0u);
  o.code_bits = 0;
  for (uint64_t s = 0; s < o.segments; ++s) {
    uint64_t words = (seg_bits[s] + 31) / 32;
    o.seg_off[s + 1] = (uint32_t)(o.seg_off[s] + words);
    o.code_bits += seg_bits[s];
  }
  o.stream_words = o.seg_off[o.segments];
  o.stream.assign(o.stream_words + 2, 0u);
  for (uint64_t s = 0; s < o.segments; ++s) {
    BitWriter bw{&o.stream, o.seg_off[s]};
    uint64_t g_end = std::min<uint64_t>((s + 1) * seg_groups, o.groups);
    for (uint64_t g = s * seg_groups; g < g_end; ++g) {
      if (group_is_verbatim(o, g)) continue;
      for (int j = 0; j < kGroup; ++j) {
        int slot = o.slot_of[exponent_of(w[g * kGroup + j])];
        bw.put(o.code[slot], o.code_len[slot]);
      }
    }
  }

  // verbatim store: raw exponents of each verbatim group, in group order
  o.vexp.clear();
  for (uint64_t g = 0; g < o.groups; ++g) {
    if (!group_is_verbatim(o, g)) continue;
    for (int j = 0; j < kGroup; ++j) o.vexp.push_back(exponent_of(w[g * kGroup + j]));
  }
  return UWO_OK;
}

// Canonical decoding one bit at a time: after reading l bits the code value c
// is a complete codeword of length l exactly when it lies in
// [first[l], first[l] + count[l]).
int decode_exponents(const Oracle& o, uint8_t* e_out) {
  int count[kLMax + 1] = {0};
  for (int s = 0; s < kPalette; ++s)
    if (o.code_len[s] > 0) count[o.code_len[s]]++;
  // first[l] = smallest codeword of length l (the same recurrence as the
  // assignment: first[1] = 0, first[l] = (first[l-1] + count[l-1]) << 1)
  int first[kLMax + 1] = {0};
  int offset[kLMax + 1] = {0};
  {
    int idx = 0;
    for (int l = 1; l <= kLMax; ++l) {
      first[l] = l == 1 ? 0 : (first[l - 1] + count[l - 1]) << 1;
      offset[l] = idx;
      idx += count[l];
    }
  }
  // symbols ordered by (length, slot): canonical order
  std::vector<int> ordered;
  for (int l = 1; l <= kLMax; ++l)
    for (int s = 0; s < kPalette; ++s)
      if (o.code_len[s] == l) ordered.push_back(s);

  for (uint64_t s = 0; s < o.segments; ++s) {
    uint64_t word0 = o.seg_off[s], word1 = o.seg_off[s + 1];
    uint64_t limit_bits = (word1 - word0) * 32;
    uint64_t bitpos = 0;
    uint64_t g_end = std::min<uint64_t>((s + 1) * o.seg_groups, o.groups);
    for (uint64_t g = s * o.seg_groups; g < g_end; ++g) {
      if (group_is_verbatim(o, g)) {
        uint64_t r = verbatim_rank(o, g);
        for (int j = 0; j < kGroup; ++j) e_out[g * kGroup + j] = o.vexp[r * kGroup + (uint64_t)j];
        continue;
      }
      for (int j = 0; j < kGroup; ++j) {
        int c = 0, l = 0, slot = -1;
        while (slot < 0) {
          if (l == kLMax) return UWO_ERR_CORRUPT;        // no codeword matched
          if (bitpos >= limit_bits) return UWO_ERR_CORRUPT;  // ran past the segment
          uint32_t wd = o.stream[word0 + bitpos / 32];
          int bit = (int)((wd >> (31 - (int)(bitpos % 32))) & 1u);
          ++bitpos;
          c = (c << 1) | bit;
          ++l;
          if (c - first[l] < count[l] && c >= first[l]) slot = ordered[(size_t)(offset[l] + c - first[l])];
        }
        e_out[g * kGroup + j] = o.palette[slot];
      }
    }
    // segments are word aligned: no whole unused word may follow the codes
    if (word1 > word0 && bitpos <= (word1 - word0 - 1) * 32) return UWO_ERR_CORRUPT;
    if (word1 == word0 && bitpos != 0) return UWO_ERR_CORRUPT;
  }
  return UWO_OK;
}

int decode_full(const Oracle& o, uint16_t* w_out) {
  if (o.fp8) return UWO_ERR_UNSUPPORTED;
  std::vector<uint8_t> e(o.numel);
  int st = decode_exponents(o, e.data());
  if (st != UWO_OK) return st;
  for (uint64_t i = 0; i < o.numel; ++i) w_out[i] = rebuild(o.sm[i], e[i]);
  return UWO_OK;
}

// UWF8: the same coding applied to the E4M3 exponent field.  Each weight's
// exponent field is placed where a BF16 exponent byte sits (sign and mantissa
// bits left zero; the sign+mantissa section is replaced below), so the
// histogram, palette, flags, code and stream are exactly those steps over the
// field.  The kept section becomes the packed sign+mantissa nibbles.
int compress_fp8(const uint8_t* w, uint64_t rows, uint64_t cols, uint32_t seg_groups,
                 uint32_t layout, Oracle& o) {
  if (w == nullptr || rows == 0 || cols == 0) return UWO_ERR_INVALID;
  const uint64_t numel = rows * cols;
  std::vector<uint16_t> field(numel);
  for (uint64_t i = 0; i < numel; ++i) field[i] = (uint16_t)((uint16_t)fp8_exponent_of(w[i]) << 7);
  int st = compress(field.data(), rows, cols, seg_groups, layout, o);
  if (st != UWO_OK) return st;
  o.sm.assign(numel / 2, 0);   // numel is a multiple of 64
  for (uint64_t i = 0; i < numel; ++i) {
    uint8_t nib = fp8_sign_mantissa_of(w[i]);
    o.sm[i / 2] = (uint8_t)(o.sm[i / 2] | (i % 2 == 0 ? nib : (uint8_t)(nib << 4)));
  }
  o.fp8 = true;
  return UWO_OK;
}

int decode_fp8(const Oracle& o, uint8_t* w_out) {
  if (!o.fp8) return UWO_ERR_UNSUPPORTED;
  std::vector<uint8_t> e(o.numel);
  int st = decode_exponents(o, e.data());
  if (st != UWO_OK) return st;
  for (uint64_t i = 0; i < o.numel; ++i) {
    uint8_t nib = (uint8_t)(i % 2 == 0 ? (o.sm[i / 2] & 0xF) : (o.sm[i / 2] >> 4));
    w_out[i] = fp8_rebuild(nib, e[i]);
  }
  return UWO_OK;
}

// 4-bit palette index per element, element 2i in the low nibble of byte i;
// verbatim groups give index 0 ([EVC] "四種執行管道", palette transcode).
int transcode(const Oracle& o, uint8_t* idx_out) {
  std::vector<uint8_t> e(o.numel);
  int st = decode_exponents(o, e.data());
  if (st != UWO_OK) return st;
  for (uint64_t i = 0; i < o.numel / 2; ++i) {
    uint64_t g = (2 * i) / kGroup;
    if (group_is_verbatim(o, g)) {
      idx_out[i] = 0;
      continue;
    }
    int lo = o.slot_of[e[2 * i]];
    int hi = o.slot_of[e[2 * i + 1]];
    idx_out[i] = (uint8_t)(lo | (hi << 4));
  }
  return UWO_OK;
}

// ---- UWF1 serialisation -------------------------------------------------------
// Header (2304 bytes, little-endian), then the six sections in the order
// sm, vflags, vrank, vexp, seg_off, stream, each padded with zeros to a
// multiple of 256 bytes.
constexpr uint64_t kHeaderBytes = 2304;

void put_u32(std::vector<uint8_t>& b, uint64_t at, uint32_t v) {
  for (int i = 0; i < 4; ++i) b[at + (uint64_t)i] = (uint8_t)(v >> (8 * i));
}
void put_u64(std::vector<uint8_t>& b, uint64_t at, uint64_t v) {
  for (int i = 0; i < 8; ++i) b[at + (uint64_t)i] = (uint8_t)(v >> (8 * i));
}
uint64_t pad256(uint64_t n) { return (n + 255) / 256 * 256; }

std::vector<uint8_t> serialise(const Oracle& o) {
  uint64_t sizes[6] = {o.numel, 4 * o.flag_words, 4 * o.flag_words, (uint64_t)o.vexp.size(),
                       4 * (o.segments + 1), 4 * (o.stream_words + 2)};
  uint64_t total = kHeaderBytes;
  for (uint64_t s : sizes) total += pad256(s);
  std::vector<uint8_t> b(total, 0);
  b[0] = 'U'; b[1] = 'W'; b[2] = 'F'; b[3] = '1';
  put_u32(b, 4, 1);                // version
  put_u32(b, 8, o.layout);
  put_u32(b, 12, o.seg_groups);
  put_u64(b, 16, o.rows);
  put_u64(b, 24, o.cols);
  put_u32(b, 32, o.palette_size);
  put_u32(b, 36, o.n_coded);
  for (int i = 0; i < 16; ++i) b[40 + (uint64_t)i] = o.palette[i];
  for (int i = 0; i < 16; ++i) b[56 + (uint64_t)i] = o.code_len[i];
  put_u64(b, 72, o.verbatim_groups);
  put_u64(b, 80, o.stream_words);
  for (int v = 0; v < 256; ++v) put_u64(b, 88 + 8 * (uint64_t)v, o.hist[v]);
  for (int s = 0; s < 16; ++s) put_u64(b, 2136 + 8 * (uint64_t)s, o.coded_count[s]);
  uint64_t at = kHeaderBytes;
  const uint8_t* srcs[6] = {o.sm.data(), (const uint8_t*)o.vflags.data(),
                            (const uint8_t*)o.vrank.data(), o.vexp.data(),
                            (const uint8_t*)o.seg_off.data(), (const uint8_t*)o.stream.data()};
  for (int k = 0; k < 6; ++k) {
    // sections of 32-bit words are written byte by byte, least significant first
    if (k == 0 || k == 3) {
      for (uint64_t i = 0; i < sizes[k]; ++i) b[at + i] = srcs[k][i];
    } else {
      const std::vector<uint32_t>* vec = k == 1 ? &o.vflags : k == 2 ? &o.vrank
                                       : k == 4 ? &o.seg_off : &o.stream;
      for (uint64_t i = 0; i < vec->size(); ++i) put_u32(b, at + 4 * i, (*vec)[i]);
    }
    at += pad256(sizes[k]);
  }
  return b;
}

// ---- GEMM reference ([EVC] "重建矩陣乘法核心運作") ---------------------------
// The reconstructive matmul computes the product a matmul on the uncompressed
// weights gives: y = x . W^T.  The reference is that definition in fp64 on the
// ORIGINAL bf16 weights, k ascending:
//   y[b][n] = sum_k x[b][k] * W[n][k],   A[b][n] = sum_k |x[b][k] * W[n][k]|,
// where W[n][k] = stored[n][k] (layout 0) or stored[k][n] (layout 1).  A is the
// magnitude the acceptance bound |y_gpu - y| <= 2^-10 * A scales with.

// Exact widening of a bf16 bit pattern: the pattern is the top half of the
// fp32 with the same value, and every fp32 is exact in fp64.
inline double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Columns cols[0..ncols) of y and A (row-major [batch][ncols]); every column
// when cols is null (ncols must then be N).
int gemm_ref(const uint16_t* x, uint64_t batch, uint64_t K, const uint16_t* stored, uint64_t N,
             uint32_t layout, const int64_t* cols, uint64_t ncols, double* y, double* A) {
  if (!x || !stored || !y || !A || layout > 1) return UWO_ERR_INVALID;
  std::vector<double> wrow(K);
  for (uint64_t j = 0; j < ncols; ++j) {
    const uint64_t n = cols ? (uint64_t)cols[j] : j;
    if (n >= N) return UWO_ERR_INVALID;
    for (uint64_t k = 0; k < K; ++k)
      wrow[k] = bf16_value(layout == 0 ? stored[n * K + k] : stored[k * N + n]);
    for (uint64_t b = 0; b < batch; ++b) {
      double sum = 0.0, mag = 0.0;
      for (uint64_t k = 0; k < K; ++k) {
        const double p = bf16_value(x[b * K + k]) * wrow[k];
        sum += p;
        mag += std::fabs(p);
      }
      y[b * ncols + j] = sum;
      A[b * ncols + j] = mag;
    }
  }
  return UWO_OK;
}

}  // namespace

// ---- C entry points used by oracle/oracle.py ---------------------------------
extern "C" {

void* uwo_compress(const uint16_t* w, uint64_t rows, uint64_t cols, uint32_t seg_groups,
                   uint32_t layout, int* status) {
  Oracle* o = new (std::nothrow) Oracle();
  if (o == nullptr) {
    if (status) *status = UWO_ERR_NOMEM;
    return nullptr;
  }
  int st = compress(w, rows, cols, seg_groups, layout, *o);
  if (status) *status = st;
  if (st != UWO_OK) {
    delete o;
    return nullptr;
  }
  return o;
}

void* uwo_compress_fp8(const uint8_t* w, uint64_t rows, uint64_t cols, uint32_t seg_groups,
                       uint32_t layout, int* status) {
  Oracle* o = new (std::nothrow) Oracle();
  if (o == nullptr) {
    if (status) *status = UWO_ERR_NOMEM;
    return nullptr;
  }
  int st = compress_fp8(w, rows, cols, seg_groups, layout, *o);
  if (status) *status = st;
  if (st != UWO_OK) {
    delete o;
    return nullptr;
  }
  return o;
}

int uwo_decode_fp8(const void* h, uint8_t* out) {
  return decode_fp8(*static_cast<const Oracle*>(h), out);
}

void uwo_free(void* h) { delete static_cast<Oracle*>(h); }

// scalars: rows, cols, numel, groups, segments, flag_words, seg_groups, layout,
// palette_size, n_coded, V, W, code_bits, vexp_bytes
int uwo_scalars(const void* h, uint64_t* out14) {
  const Oracle* o = static_cast<const Oracle*>(h);
  if (!o || !out14) return UWO_ERR_INVALID;
  uint64_t v[14] = {o->rows, o->cols, o->numel, o->groups, o->segments, o->flag_words,
                    o->seg_groups, o->layout, o->palette_size, o->n_coded,
                    o->verbatim_groups, o->stream_words, o->code_bits, (uint64_t)o->vexp.size()};
  std::memcpy(out14, v, sizeof(v));
  return UWO_OK;
}

int uwo_tables(const void* h, uint8_t* palette16, uint8_t* len16, uint16_t* code16,
               uint64_t* hist256, uint64_t* coded16) {
  const Oracle* o = static_cast<const Oracle*>(h);
  if (!o) return UWO_ERR_INVALID;
  std::memcpy(palette16, o->palette, 16);
  std::memcpy(len16, o->code_len, 16);
  std::memcpy(code16, o->code, 32);
  std::memcpy(hist256, o->hist, 256 * 8);
  std::memcpy(coded16, o->coded_count, 16 * 8);
  return UWO_OK;
}

// section ids: 0 sm, 1 vflags, 2 vrank, 3 vexp, 4 seg_off, 5 stream
int uwo_section(const void* h, int id, const void** ptr, uint64_t* bytes) {
  const Oracle* o = static_cast<const Oracle*>(h);
  if (!o || !ptr || !bytes) return UWO_ERR_INVALID;
  switch (id) {
    case 0: *ptr = o->sm.data(); *bytes = o->sm.size(); break;
    case 1: *ptr = o->vflags.data(); *bytes = 4 * o->vflags.size(); break;
    case 2: *ptr = o->vrank.data(); *bytes = 4 * o->vrank.size(); break;
    case 3: *ptr = o->vexp.data(); *bytes = o->vexp.size(); break;
    case 4: *ptr = o->seg_off.data(); *bytes = 4 * o->seg_off.size(); break;
    case 5: *ptr = o->stream.data(); *bytes = 4 * o->stream.size(); break;
    default: return UWO_ERR_INVALID;
  }
  return UWO_OK;
}

// Overwrite one section word (used by tests to plant corruption in the oracle).
int uwo_poke_u32(void* h, int id, uint64_t index, uint32_t value) {
  Oracle* o = static_cast<Oracle*>(h);
  std::vector<uint32_t>* v = id == 1 ? &o->vflags : id == 2 ? &o->vrank
                           : id == 4 ? &o->seg_off : id == 5 ? &o->stream : nullptr;
  if (!v || index >= v->size()) return UWO_ERR_INVALID;
  (*v)[index] = value;
  return UWO_OK;
}

int uwo_decode_exponent(const void* h, uint8_t* out) {
  return decode_exponents(*static_cast<const Oracle*>(h), out);
}
int uwo_decode_full(const void* h, uint16_t* out) {
  return decode_full(*static_cast<const Oracle*>(h), out);
}
int uwo_transcode(const void* h, uint8_t* out) {
  return transcode(*static_cast<const Oracle*>(h), out);
}

// Serialised UWF1 blob; cap == 0 returns the size only.
uint64_t uwo_export(const void* h, uint8_t* buf, uint64_t cap) {
  if (static_cast<const Oracle*>(h)->fp8) return 0;   // UWF1 is the BF16 format only
  std::vector<uint8_t> b = serialise(*static_cast<const Oracle*>(h));
  if (buf != nullptr && cap >= b.size()) std::memcpy(buf, b.data(), b.size());
  return b.size();
}

int uwo_package_merge(const uint64_t* weights, int n, int lmax, uint8_t* len_out) {
  return package_merge(weights, n, lmax, len_out) ? UWO_OK : UWO_ERR_INVALID;
}

int uwo_canonical(const uint8_t* len, int n, uint16_t* code_out) {
  canonical_codes(len, n, code_out);
  return UWO_OK;
}

int uwo_gemm_ref(const uint16_t* x, uint64_t batch, uint64_t K, const uint16_t* stored, uint64_t N,
                 uint32_t layout, const int64_t* cols, uint64_t ncols, double* y, double* A) {
  return gemm_ref(x, batch, K, stored, N, layout, cols, ncols, y, A);
}

}  // extern "C"
