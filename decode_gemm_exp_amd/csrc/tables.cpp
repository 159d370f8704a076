// tables.cpp -- the small per-matrix tables: palette, code lengths, canonical
// codes and the decoder's lookup table.  All of it is O(256) host work done
// once per matrix; the per-weight passes run on the GPU.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736), cited by section heading.
#include <algorithm>
#include <cstring>

#include "uw_internal.h"

namespace uw {

// The 16 most frequent exponents ([EVC] "BF16權重壓縮原理"), ties broken
// toward the smaller exponent, kept in ascending order so that slot order is
// exponent order.
void choose_palette(Tables& t) {
  bool taken[256] = {};
  int chosen = 0;
  while (chosen < kPal) {
    int best = -1;
    for (int v = 0; v < 256; ++v) {
      if (taken[v] || t.hist[v] == 0) continue;
      if (best < 0 || t.hist[v] > t.hist[best]) best = v;   // strict: first (smallest) wins ties
    }
    if (best < 0) break;
    taken[best] = true;
    ++chosen;
  }
  t.palette_size = (uint32_t)chosen;
  std::memset(t.palette, 0, sizeof(t.palette));
  for (int v = 0; v < 256; ++v) t.slot_of[v] = -1;
  int slot = 0;
  for (int v = 0; v < 256; ++v)
    if (taken[v]) {
      t.palette[slot] = (uint8_t)v;
      t.slot_of[v] = (int16_t)slot;
      ++slot;
    }
}

// Length-limited optimal code lengths by package-merge (Larmore & Hirschberg,
// JACM 1990).  Each list item carries its weight and how many times every
// symbol occurs inside it; leaves sort by (weight, symbol) and precede
// packages of equal weight.
namespace {
struct Node {
  uint64_t weight;
  uint8_t mult[kPal];
};
}  // namespace

bool limited_lengths(const uint64_t* w, int n, int lmax, uint8_t* len) {
  if (n < 2 || n > kPal || (1 << lmax) < n) return false;
  Node leaves[kPal];
  int order[kPal];
  for (int i = 0; i < n; ++i) order[i] = i;
  std::sort(order, order + n, [&](int a, int b) { return w[a] != w[b] ? w[a] < w[b] : a < b; });
  for (int i = 0; i < n; ++i) {
    std::memset(&leaves[i], 0, sizeof(Node));
    leaves[i].weight = w[order[i]];
    leaves[i].mult[order[i]] = 1;
  }
  // a list never exceeds 2n - 1 items (n leaves + at most n - 1 packages)
  Node cur[2 * kPal], nxt[2 * kPal];
  int cur_n = n;
  std::memcpy(cur, leaves, sizeof(Node) * (size_t)n);
  for (int level = 1; level < lmax; ++level) {
    int pk = cur_n / 2;   // packages are pairs (cur[2i], cur[2i+1])
    int a = 0, b = 0, out = 0;
    while (a < n || b < pk) {
      bool leaf;
      if (a == n) leaf = false;
      else if (b == pk) leaf = true;
      else leaf = leaves[a].weight <= cur[2 * b].weight + cur[2 * b + 1].weight;
      if (leaf) {
        nxt[out++] = leaves[a++];
      } else {
        Node p;
        p.weight = cur[2 * b].weight + cur[2 * b + 1].weight;
        for (int s = 0; s < kPal; ++s) p.mult[s] = (uint8_t)(cur[2 * b].mult[s] + cur[2 * b + 1].mult[s]);
        nxt[out++] = p;
        ++b;
      }
    }
    std::memcpy(cur, nxt, sizeof(Node) * (size_t)out);
    cur_n = out;
  }
  std::memset(len, 0, (size_t)n);
  for (int i = 0; i < 2 * n - 2; ++i)
    for (int s = 0; s < n; ++s) len[s] = (uint8_t)(len[s] + cur[i].mult[s]);
  return true;
}

// Canonical codes: codewords of one length are consecutive integers in slot
// order, and each length starts where the previous one ended, shifted left.
void assign_codes(Tables& t) {
  int per_len[kMaxLen + 1] = {};
  for (int s = 0; s < kPal; ++s)
    if (t.code_len[s]) per_len[t.code_len[s]]++;
  uint32_t start[kMaxLen + 2] = {};
  uint32_t c = 0;
  for (int l = 1; l <= kMaxLen; ++l) {
    start[l] = c;
    c = (c + (uint32_t)per_len[l]) << 1;
  }
  for (int s = 0; s < kPal; ++s) t.code[s] = t.code_len[s] ? (uint16_t)start[t.code_len[s]]++ : 0;
}

// Decoder table: entry v describes the 12-bit window v (first stream bit =
// bit 11): the whole codewords it starts with (up to 8), the bits they take
// and their slots, in the two-word layout of kLutWords.  A window that starts
// with no valid codeword (possible only with a one-symbol code) gets one
// codeword of one bit, slot 0 and the invalid bit, so decoders always make
// progress and can OR the entries to detect corruption.
void build_decode_lut(const Tables& t, uint32_t* lut) {
  for (uint32_t v = 0; v < (1u << kLutBits); ++v) {
    int pos = 0, cnt = 0;
    uint32_t syms = 0;
    while (cnt < 8) {
      int found = -1, flen = 0;
      for (int s = 0; s < kPal && found < 0; ++s) {
        int l = t.code_len[s];
        if (l == 0 || l > kLutBits - pos) continue;
        uint32_t bits = (v >> (kLutBits - pos - l)) & ((1u << l) - 1u);
        if (bits == t.code[s]) {
          found = s;
          flen = l;
        }
      }
      if (found < 0) break;
      syms |= (uint32_t)found << (4 * cnt);
      pos += flen;
      ++cnt;
    }
    if (cnt == 0) {
      lut[2 * v] = 1u | (4u << 8) | kLutInvalid;
      lut[2 * v + 1] = 0;
    } else {
      lut[2 * v] = (uint32_t)pos | ((uint32_t)(4 * cnt) << 8);
      lut[2 * v + 1] = syms;
    }
  }
}

}  // namespace uw
