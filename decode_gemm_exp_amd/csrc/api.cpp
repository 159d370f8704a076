// api.cpp -- the extern "C" entry points of libunweight (include/unweight.h):
// argument checks, section allocation, table construction, UWF1
// serialisation, pipeline dispatch and the CU-split sequence runner.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736), cited by section heading.
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>
#include <tuple>
#include <set>

#include "uw_internal.h"

using namespace uw;

int uw::device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cached[dev] = c;
  }
  return cached[dev];
}

hipError_t uw::allow_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::tuple<const void*, int, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kernel, dev, bytes);
  if (done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert(key);
  return e;
}

namespace {

#define UW_HIP(call)                                   \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) {                            \
      if (std::getenv("UW_LOG"))                       \
        std::fprintf(stderr, "unweight: %s failed: %s (%s:%d)\n", #call, hipGetErrorString(e_), \
                     __FILE__, __LINE__);              \
      return e_ == hipErrorOutOfMemory ? UW_ERR_NOMEM : e_ == hipErrorNotSupported ? UW_ERR_UNSUPPORTED \
                                                                                 : UW_ERR_DEVICE; \
    }                                                  \
  } while (0)

#define UW_CHECK(st)             \
  do {                           \
    uw_status s_ = (st);         \
    if (s_ != UW_OK) return s_;  \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline uint64_t pad256(uint64_t n) { return (n + 255) / 256 * 256; }

// device memory through allocator a (uw_set_allocator's hooks, or hipMalloc)
template <typename T>
uw_status dev_alloc(const uw_allocator& a, T** p, uint64_t bytes) {
  void* q = nullptr;
  const uw_status st = alloc_with(a, &q, bytes);
  *p = static_cast<T*>(q);
  return st;
}

template <typename T>
void dev_free(const uw_allocator& a, T*& p) {
  if (p) free_with(a, (void*)p);
  p = nullptr;
}

void free_sections(uw_matrix* m) {
  const uw_allocator a = m->alloc;
  dev_free(a, m->sm);
  dev_free(a, m->vflags);
  dev_free(a, m->vrank);
  dev_free(a, m->vexp);
  dev_free(a, m->seg_off);
  dev_free(a, m->stream);
  dev_free(a, m->lut);
  dev_free(a, m->pidx);
  dev_free(a, m->corrupt);
}

// Stream allocation: W + 2 words, rounded up so that the decoder's aligned
// 16-byte chunk loads (up to 8 words past a segment) stay inside it.
uint64_t stream_alloc_words(uint64_t W) { return (W + 2 + 3) / 4 * 4 + 8; }

bool valid_seg_groups(uint32_t sg) { return sg >= 1 && sg <= 64 && (sg & (sg - 1)) == 0; }

void shape_from(uw_matrix* m, uint64_t rows, uint64_t cols, uint32_t layout, uint32_t sg) {
  m->rows = rows;
  m->cols = cols;
  m->layout = layout;
  m->seg_groups = sg;
  m->numel = rows * cols;
  m->groups = m->numel / kGroup;
  m->segments = (m->groups + sg - 1) / sg;
  m->flag_words = (m->groups + 31) / 32;
}

uint64_t logical_n(const uw_matrix* m) { return m->layout == 0 ? m->rows : m->cols; }
uint64_t logical_k(const uw_matrix* m) { return m->layout == 0 ? m->cols : m->rows; }

// derive code lengths and codes from the coded histogram
void finish_code(Tables& t) {
  std::memset(t.code_len, 0, sizeof(t.code_len));
  int idx[kPal], n = 0;
  uint64_t wts[kPal];
  for (int s = 0; s < kPal; ++s)
    if (t.coded_count[s] > 0) {
      idx[n] = s;
      wts[n] = t.coded_count[s];
      ++n;
    }
  t.n_coded = (uint32_t)n;
  if (n == 1) {
    t.code_len[idx[0]] = 1;
  } else if (n >= 2) {
    uint8_t lens[kPal];
    limited_lengths(wts, n, kMaxLen, lens);
    for (int i = 0; i < n; ++i) t.code_len[idx[i]] = lens[i];
  }
  assign_codes(t);
}

uint64_t len_pack(const Tables& t) {
  uint64_t p = 0;
  for (int s = 0; s < kPal; ++s) p |= (uint64_t)(t.code_len[s] & 15u) << (4 * s);
  return p;
}

void pal_words(const Tables& t, PalView* out) {
  for (int i = 0; i < 4; ++i)
    out->w[i] = (uint32_t)t.palette[4 * i] | ((uint32_t)t.palette[4 * i + 1] << 8) |
                ((uint32_t)t.palette[4 * i + 2] << 16) | ((uint32_t)t.palette[4 * i + 3] << 24);
  // slots >= palette_size never occur outside verbatim groups, so a run of
  // palette_size consecutive exponents decodes as slot + first entry
  const uint32_t ps = t.palette_size;
  out->run = ps > 0 && (uint32_t)t.palette[ps - 1] - (uint32_t)t.palette[0] == ps - 1 &&
             (uint32_t)t.palette[0] + 15u <= 255u;
  out->base4 = out->run ? 0x01010101u * (uint32_t)t.palette[0] : 0u;
}

uw_status upload_lut(uw_matrix* m, hipStream_t s) {
  std::vector<uint32_t> lut((size_t)kLutWords << kLutBits);
  build_decode_lut(m->t, lut.data());
  if (!m->lut) UW_CHECK(dev_alloc(m->alloc, &m->lut, lut.size() * 4));
  UW_HIP(hipMemcpyAsync(m->lut, lut.data(), lut.size() * 4, hipMemcpyHostToDevice, s));
  UW_HIP(hipStreamSynchronize(s));
  return UW_OK;
}

uint64_t sm_bytes(const uw_matrix* m) { return m->fp8 ? m->numel / 2 : m->numel; }

uint64_t compressed_bytes(const uw_matrix* m) {
  return kHeaderBytes + sm_bytes(m) + 8 * m->flag_words + 64 * m->V + 4 * (m->segments + 1) + 4 * (m->W + 2);
}

uint64_t export_bytes(const uw_matrix* m) {
  return kHeaderBytes + pad256(m->numel) + 2 * pad256(4 * m->flag_words) + pad256(64 * m->V) +
         pad256(4 * (m->segments + 1)) + pad256(4 * (m->W + 2));
}

void wr32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }
void wr64(uint8_t* p, uint64_t v) { std::memcpy(p, &v, 8); }
uint32_t rd32(const uint8_t* p) { uint32_t v; std::memcpy(&v, p, 4); return v; }
uint64_t rd64(const uint8_t* p) { uint64_t v; std::memcpy(&v, p, 8); return v; }

// UWF1 header offsets
enum : uint32_t {
  kOffMagic = 0, kOffVersion = 4, kOffLayout = 8, kOffSegGroups = 12, kOffRows = 16, kOffCols = 24,
  kOffPalSize = 32, kOffNCoded = 36, kOffPalette = 40, kOffLen = 56, kOffV = 72, kOffW = 80,
  kOffHist = 88, kOffCoded = 2136
};

// ---- preprocessing + GEMM of one matrix -------------------------------------------------
size_t prep_bytes(const uw_matrix* m, int p) {
  switch (p) {
    case UW_PIPE_FULL: return pad256(2 * m->numel);
    case UW_PIPE_EXPONENT: return pad256(m->numel);
    case UW_PIPE_PALETTE_TRANSCODE: return pad256(m->numel / 2);
    default: return 0;
  }
}

WeightView base_view(const uw_matrix* m) {
  WeightView v;
  std::memset(&v, 0, sizeof(v));
  v.layout = (int)m->layout;
  v.n = logical_n(m);
  v.k = logical_k(m);
  v.sm = m->sm;
  v.vflags = m->vflags;
  v.vrank = m->vrank;
  v.vexp = m->vexp;
  v.vexp_bytes = 64 * m->V;
  pal_words(m->t, &v.pal);
  return v;
}

DecodeArgs decode_args(const uw_matrix* m, void* out) {
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.stream = m->stream;
  a.stream_words = stream_alloc_words(m->W);
  a.seg_off = m->seg_off;
  a.vflags = m->vflags;
  a.vrank = m->vrank;
  a.vexp = m->vexp;
  a.vexp_bytes = 64 * m->V;
  a.sm = m->sm;
  a.lut = m->lut;
  pal_words(m->t, &a.pal);
  a.len_pack = len_pack(m->t);
  a.groups = m->groups;
  a.segments = m->segments;
  a.seg_groups = m->seg_groups;
  a.wave_span = m->wave_span;
  a.out = out;
  a.corrupt = m->corrupt;
  return a;
}

uw_status preprocess(const uw_matrix* m, int p, void* buf, hipStream_t s) {
  if (p == UW_PIPE_PALETTE_DIRECT) return m->pidx ? UW_OK : UW_ERR_STATE;
  if (!m->stream) return UW_ERR_STATE;
  const int mode = p == UW_PIPE_FULL ? kDecodeFull : p == UW_PIPE_EXPONENT ? kDecodeExponent : kDecodeNibble;
  UW_HIP(launch_decode(decode_args(m, buf), mode, s));
  return UW_OK;
}

WeightView pipeline_view(const uw_matrix* m, int p, const void* buf) {
  WeightView v = base_view(m);
  switch (p) {
    case UW_PIPE_FULL: v.fmt = kFmtBf16; v.bf16 = static_cast<const uint16_t*>(buf); break;
    case UW_PIPE_EXPONENT: v.fmt = kFmtExp; v.ex = static_cast<const uint8_t*>(buf); break;
    case UW_PIPE_PALETTE_TRANSCODE: v.fmt = v.pal.run ? kFmtPalRun : kFmtPal; v.pidx = static_cast<const uint8_t*>(buf); break;
    default: v.fmt = v.pal.run ? kFmtPalRun : kFmtPal; v.pidx = m->pidx; break;
  }
  return v;
}

size_t partial_bytes(const uw_matrix* m, int p, int64_t batch, const uw_kernel_cfg* cfg) {
  WeightView v = pipeline_view(m, p, nullptr);
  return pad256(gemm_partial_elems(v, batch, cfg) * sizeof(float));
}

bool pipeline_feasible(const uw_matrix* m, int p) {
  if (p == UW_PIPE_PALETTE_DIRECT) return m->pidx != nullptr;
  return p >= UW_PIPE_FULL && p <= UW_PIPE_PALETTE_TRANSCODE && m->stream != nullptr;
}

bool pipeline_arg(int p) { return (p >= UW_PIPE_FULL && p <= UW_PIPE_PALETTE_DIRECT) || p == UW_PIPE_AUTO; }

bool cfg_empty(const uw_kernel_cfg& c) { return c.variant <= 0 && c.split_k <= 0 && c.decode_cus <= 0; }

// What one call on m runs: the pipeline (UW_PIPE_AUTO resolved) and the
// kernel configuration (the caller's; without one, the tuned entry's when it
// names that pipeline; else none, i.e. the library default).
struct Plan {
  int p = UW_PIPE_EXPONENT;
  uw_kernel_cfg cfg{};
  bool has_cfg = false;
  const uw_kernel_cfg* cfgp() const { return has_cfg ? &cfg : nullptr; }
};

Plan plan_call(const uw_matrix* m, int p, int64_t batch, const uw_kernel_cfg* cfg) {
  Plan r;
  uw_tune_entry e;
  const bool tuned = batch > 0 && !m->fp8 &&
                     tuned_lookup(logical_n(m), logical_k(m), (int)m->layout, residency_of(m), batch, &e);
  if (p == UW_PIPE_AUTO)
    r.p = tuned && pipeline_feasible(m, e.pipeline) ? e.pipeline
          : m->pidx ? UW_PIPE_PALETTE_DIRECT : UW_PIPE_EXPONENT;
  else
    r.p = p;
  if (cfg) {
    r.cfg = *cfg;
    r.has_cfg = true;
  } else if (tuned && e.pipeline == r.p) {
    r.cfg.variant = e.variant;
    r.cfg.split_k = e.split_k;
    r.cfg.decode_cus = e.decode_cus;
    r.cfg.reserved = 0;
    r.has_cfg = true;
  }
  return r;
}

// The pipeline a grouped call runs: the tuned one when every matrix's entry
// names the same feasible pipeline, else direct palette when every matrix
// has resident indices, else exponent.
int plan_group_pipeline(const uw_matrix* const* ms, int count, int p, int64_t batch) {
  if (p != UW_PIPE_AUTO) return p;
  int tp = -1;
  bool same = true, all_pidx = true;
  for (int i = 0; i < count; ++i) {
    const uw_matrix* m = ms[i];
    all_pidx = all_pidx && m->pidx != nullptr;
    uw_tune_entry e;
    if (!m->fp8 && tuned_lookup(logical_n(m), logical_k(m), (int)m->layout, residency_of(m), batch, &e) &&
        pipeline_feasible(m, e.pipeline)) {
      if (tp < 0) tp = e.pipeline;
      else if (tp != e.pipeline) same = false;
    } else {
      same = false;
    }
  }
  if (same && tp >= 0) return tp;
  return all_pidx ? UW_PIPE_PALETTE_DIRECT : UW_PIPE_EXPONENT;
}

// What a grouped call runs.  The group's own tuning entry (its matrix count,
// total N, K, layout and residency) decides first: its pipeline for AUTO when
// every matrix can run it, and its kernel configuration when the caller gives
// none and the call's pipeline is the entry's.  Without one, AUTO takes
// plan_group_pipeline and cfg == NULL the grouped kernels' defaults.
Plan plan_group(const uw_matrix* const* ms, int count, int p, int64_t batch, const uw_kernel_cfg* cfg) {
  Plan r;
  uw_tune_entry e;
  bool tuned = count >= 2 && count <= kTuneGroupMax && batch > 0;
  uint64_t ntot = 0;
  for (int i = 0; i < count && tuned; ++i) {
    const uw_matrix* m = ms[i];
    tuned = !m->fp8 && m->layout == ms[0]->layout && logical_k(m) == logical_k(ms[0]) &&
            residency_of(m) == residency_of(ms[0]);
    ntot += logical_n(m);
  }
  tuned = tuned && tuned_lookup(ntot, logical_k(ms[0]), (int)ms[0]->layout, residency_of(ms[0]), batch, &e, count);
  for (int i = 0; i < count && tuned; ++i) tuned = pipeline_feasible(ms[i], e.pipeline);
  if (p == UW_PIPE_AUTO)
    r.p = tuned ? e.pipeline : plan_group_pipeline(ms, count, p, batch);
  else
    r.p = p;
  if (cfg) {
    r.cfg = *cfg;
    r.has_cfg = true;
  } else if (tuned && e.pipeline == r.p) {
    r.cfg.variant = e.variant;
    r.cfg.split_k = e.split_k;
    r.cfg.decode_cus = e.decode_cus;
    r.cfg.reserved = 0;
    r.has_cfg = true;
  }
  return r;
}

uw_status check_matmul_args(const uw_matrix* m, int p, const uint16_t* x, int64_t batch, const float* y) {
  if (!m || !x || !y || batch <= 0) return UW_ERR_INVALID;
  if (m->fp8) return UW_ERR_UNSUPPORTED;   // the GEMMs rebuild BF16 weights
  if (p < UW_PIPE_FULL || p > UW_PIPE_PALETTE_DIRECT) return UW_ERR_INVALID;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(y) & 3u)) return UW_ERR_INVALID;
  if (logical_k(m) % 8 != 0) return UW_ERR_UNSUPPORTED;
  if (p == UW_PIPE_PALETTE_DIRECT && !m->pidx) return UW_ERR_STATE;
  if (p != UW_PIPE_PALETTE_DIRECT && !m->stream) return UW_ERR_STATE;
  return UW_OK;
}

}  // namespace

// =====================================================================================
extern "C" {

const char* uw_status_str(uw_status st) {
  switch (st) {
    case UW_OK: return "ok";
    case UW_ERR_INVALID: return "invalid argument";
    case UW_ERR_UNSUPPORTED: return "unsupported shape";
    case UW_ERR_NOMEM: return "out of memory";
    case UW_ERR_DEVICE: return "HIP runtime error";
    case UW_ERR_CORRUPT: return "corrupt compressed data";
    case UW_ERR_STATE: return "handle lacks the required section";
    case UW_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

uint32_t uw_version(void) { return (1u << 16) | 0u; }

}  // extern "C"

namespace {

// Arguments shared by the BF16 and FP8 compress entry points.
uw_status compress_args(const void* w_dev, int64_t n, int64_t k, uw_layout layout, const uw_compress_opts* opts,
                        uw_matrix** out, uint32_t* sg, uint64_t* rows, uint64_t* cols) {
  if (!out) return UW_ERR_INVALID;
  *out = nullptr;
  if (!w_dev || n <= 0 || k <= 0 || (layout != UW_LAYOUT_NK && layout != UW_LAYOUT_KN)) return UW_ERR_INVALID;
  if (!aligned16(w_dev)) return UW_ERR_INVALID;
  *sg = (opts && opts->seg_groups) ? opts->seg_groups : 4u;
  if (!valid_seg_groups(*sg) || (opts && opts->flags)) return UW_ERR_INVALID;
  *rows = layout == UW_LAYOUT_NK ? (uint64_t)n : (uint64_t)k;
  *cols = layout == UW_LAYOUT_NK ? (uint64_t)k : (uint64_t)n;
  if (*cols % kGroup != 0) return UW_ERR_UNSUPPORTED;
  if (*rows * *cols >= (1ull << 32)) return UW_ERR_UNSUPPORTED;
  return UW_OK;
}

// The coding passes over a device array of 16-bit words whose bits 14..7
// are the coded exponent (BF16 weights, or FP8 exponent fields placed there).
uw_status compress_words(const uint16_t* w_dev, uint64_t rows, uint64_t cols, uw_layout layout, uint32_t sg,
                         const uw_allocator& alloc, hipStream_t s, uw_matrix** out) {
  uw_matrix* m = new (std::nothrow) uw_matrix();
  if (!m) return UW_ERR_NOMEM;
  m->alloc = alloc;
  struct Guard {
    uw_matrix* m;
    uw_allocator a;
    void* scratch = nullptr;
    ~Guard() {
      if (scratch) free_with(a, scratch);
      if (m) { free_sections(m); delete m; }
    }
  } guard{m, alloc};
  UW_HIP(hipGetDevice(&m->device));
  shape_from(m, rows, cols, (uint32_t)layout, sg);

  UW_CHECK(dev_alloc(m->alloc, &m->sm, m->numel));
  UW_CHECK(dev_alloc(m->alloc, &m->vflags, 4 * m->flag_words));
  UW_CHECK(dev_alloc(m->alloc, &m->vrank, 4 * m->flag_words));
  UW_CHECK(dev_alloc(m->alloc, &m->seg_off, 4 * (m->segments + 1)));
  UW_CHECK(dev_alloc(m->alloc, &m->corrupt, sizeof(int)));
  UW_HIP(hipMemsetAsync(m->corrupt, 0, sizeof(int), s));

  // scratch: hist u32[256] | coded u32[16] | total u64 | slot/len tables | codebook u32[256] | seg words |
  // scan tile sums u64
  const uint64_t off_coded = 1024, off_total = 1088, off_slot = 1152, off_len = 1408, off_book = 1664,
                 off_seg = 2688;
  const uint64_t off_tiles = pad256(off_seg + 4 * m->segments);
  const uint64_t ntiles = scan_tiles(m->segments > m->flag_words ? m->segments : m->flag_words);
  void* scratch = nullptr;
  UW_CHECK(dev_alloc(m->alloc, &scratch, off_tiles + 8 * ntiles + 256));
  guard.scratch = scratch;
  uint8_t* sc = static_cast<uint8_t*>(scratch);
  uint32_t* d_hist = reinterpret_cast<uint32_t*>(sc);
  uint32_t* d_coded = reinterpret_cast<uint32_t*>(sc + off_coded);
  uint64_t* d_total = reinterpret_cast<uint64_t*>(sc + off_total);
  uint8_t* d_slot = sc + off_slot;
  uint8_t* d_len = sc + off_len;
  uint32_t* d_book = reinterpret_cast<uint32_t*>(sc + off_book);
  uint32_t* d_seg = reinterpret_cast<uint32_t*>(sc + off_seg);
  uint64_t* d_tiles = reinterpret_cast<uint64_t*>(sc + off_tiles);

  // 1. exponent histogram
  UW_HIP(hipMemsetAsync(sc, 0, off_slot, s));
  UW_HIP(launch_histogram(w_dev, m->numel, d_hist, s));
  uint32_t hist32[256];
  UW_HIP(hipMemcpyAsync(hist32, d_hist, sizeof(hist32), hipMemcpyDeviceToHost, s));
  UW_HIP(hipStreamSynchronize(s));
  for (int v = 0; v < 256; ++v) m->t.hist[v] = hist32[v];

  // 2. palette, verbatim flags, sign/mantissa, coded histogram, ranks
  choose_palette(m->t);
  uint8_t slot_tab[256];
  for (int v = 0; v < 256; ++v) slot_tab[v] = m->t.slot_of[v] < 0 ? 0xFFu : (uint8_t)m->t.slot_of[v];
  UW_HIP(hipMemcpyAsync(d_slot, slot_tab, 256, hipMemcpyHostToDevice, s));
  UW_HIP(launch_flags(w_dev, m->numel, m->groups, d_slot, m->sm, m->vflags, d_coded, s));
  UW_HIP(launch_rank_scan(m->vflags, m->flag_words, m->vrank, d_total, d_tiles, s));
  uint32_t coded32[16];
  uint64_t vtotal = 0;
  UW_HIP(hipMemcpyAsync(coded32, d_coded, sizeof(coded32), hipMemcpyDeviceToHost, s));
  UW_HIP(hipMemcpyAsync(&vtotal, d_total, sizeof(vtotal), hipMemcpyDeviceToHost, s));
  UW_HIP(hipStreamSynchronize(s));
  m->V = vtotal;
  for (int i = 0; i < kPal; ++i) m->t.coded_count[i] = coded32[i];
  finish_code(m->t);
  UW_CHECK(dev_alloc(m->alloc, &m->vexp, 64 * m->V));

  // 3. segment lengths and offsets
  uint8_t len_tab[256];
  uint32_t book[256];
  for (int v = 0; v < 256; ++v) {
    const int sl = m->t.slot_of[v];
    len_tab[v] = sl < 0 ? 0 : m->t.code_len[sl];
    book[v] = sl < 0 ? 0u : ((uint32_t)m->t.code[sl] << 8) | m->t.code_len[sl];
  }
  UW_HIP(hipMemcpyAsync(d_len, len_tab, 256, hipMemcpyHostToDevice, s));
  UW_HIP(hipMemcpyAsync(d_book, book, sizeof(book), hipMemcpyHostToDevice, s));
  UW_HIP(hipMemsetAsync(d_seg, 0, 4 * m->segments, s));
  UW_HIP(launch_segment_bits(w_dev, m->groups, sg, m->segments, d_len, m->vflags, d_seg, s));
  UW_HIP(launch_offsets_scan(d_seg, m->segments, m->seg_off, d_tiles, s));
  UW_HIP(hipMemsetAsync(d_coded, 0, 4, s));
  UW_HIP(launch_wave_span(m->seg_off, m->segments, d_coded, s));
  uint32_t W32 = 0, span32 = 0;
  UW_HIP(hipMemcpyAsync(&W32, m->seg_off + m->segments, 4, hipMemcpyDeviceToHost, s));
  UW_HIP(hipMemcpyAsync(&span32, d_coded, 4, hipMemcpyDeviceToHost, s));
  UW_HIP(hipStreamSynchronize(s));
  m->W = W32;
  m->wave_span = span32;

  // 4. encode
  const uint64_t sw = stream_alloc_words(m->W);
  UW_CHECK(dev_alloc(m->alloc, &m->stream, 4 * sw));
  UW_HIP(hipMemsetAsync(m->stream, 0, 4 * sw, s));
  UW_HIP(launch_encode(w_dev, m->groups, sg, m->segments, d_book, m->vflags, m->vrank, m->seg_off, m->stream,
                       m->vexp, s));
  m->code_bits = 0;
  for (int i = 0; i < kPal; ++i) m->code_bits += m->t.coded_count[i] * m->t.code_len[i];
  UW_CHECK(upload_lut(m, s));   // synchronises: host tables above stay alive until here
  guard.m = nullptr;
  *out = m;
  return UW_OK;
}

}  // namespace

extern "C" {

uw_status uw_compress(const uint16_t* w_dev, int64_t n, int64_t k, uw_layout layout,
                      const uw_compress_opts* opts, void* stream, uw_matrix** out) try {
  uint32_t sg = 0;
  uint64_t rows = 0, cols = 0;
  UW_CHECK(compress_args(w_dev, n, k, layout, opts, out, &sg, &rows, &cols));
  return compress_words(w_dev, rows, cols, layout, sg, current_allocator(), static_cast<hipStream_t>(stream), out);
} catch (...) {
  return UW_ERR_NOMEM;
}

uw_status uw_compress_fp8(const uint8_t* w_dev, int64_t n, int64_t k, uw_layout layout,
                          const uw_compress_opts* opts, void* stream, uw_matrix** out) try {
  uint32_t sg = 0;
  uint64_t rows = 0, cols = 0;
  UW_CHECK(compress_args(w_dev, n, k, layout, opts, out, &sg, &rows, &cols));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint64_t numel = rows * cols;
  const uw_allocator alloc = current_allocator();
  struct Temp {
    uw_allocator a;
    uint16_t* fields = nullptr;
    uint8_t* nib = nullptr;
    ~Temp() {
      dev_free(a, fields);
      dev_free(a, nib);
    }
  } t{alloc};
  UW_CHECK(dev_alloc(alloc, &t.fields, 2 * numel));
  UW_CHECK(dev_alloc(alloc, &t.nib, numel / 2));
  UW_HIP(launch_fp8_fields(w_dev, numel, t.fields, s));
  UW_HIP(launch_fp8_pack(w_dev, numel, t.nib, s));
  uw_matrix* m = nullptr;
  UW_CHECK(compress_words(t.fields, rows, cols, layout, sg, alloc, s, &m));   // synchronises at its end
  dev_free(m->alloc, m->sm);   // the byte section of the field array: replaced by the nibbles
  m->sm = t.nib;
  t.nib = nullptr;
  m->fp8 = true;
  *out = m;
  return UW_OK;
} catch (...) {
  return UW_ERR_NOMEM;
}

uw_status uw_get_info(const uw_matrix* m, uw_info* o) {
  if (!m || !o) return UW_ERR_INVALID;
  std::memset(o, 0, sizeof(*o));
  o->layout = m->layout;
  o->seg_groups = m->seg_groups;
  o->rows = m->rows;
  o->cols = m->cols;
  o->n = logical_n(m);
  o->k = logical_k(m);
  o->numel = m->numel;
  o->groups = m->groups;
  o->segments = m->segments;
  o->palette_size = m->t.palette_size;
  o->n_coded = m->t.n_coded;
  std::memcpy(o->palette, m->t.palette, 16);
  std::memcpy(o->code_len, m->t.code_len, 16);
  std::memcpy(o->code, m->t.code, sizeof(o->code));
  std::memcpy(o->hist, m->t.hist, sizeof(o->hist));
  std::memcpy(o->coded_count, m->t.coded_count, sizeof(o->coded_count));
  o->verbatim_groups = m->V;
  o->stream_words = m->W;
  o->code_bits = m->code_bits;
  o->compressed_bytes = compressed_bytes(m);
  o->export_bytes = export_bytes(m);
  o->bits_per_weight = 8.0 * (double)o->compressed_bytes / (double)m->numel;
  o->has_stream = m->stream != nullptr;
  o->has_palette_idx = m->pidx != nullptr;
  o->element_bits = m->fp8 ? 8 : 16;
  return UW_OK;
}

uw_status uw_export(const uw_matrix* m, void* host_buf, size_t cap, size_t* bytes) try {
  if (m && m->fp8) return UW_ERR_UNSUPPORTED;   // UWF1 carries BF16 matrices
  if (!m || !bytes) return UW_ERR_INVALID;
  const uint64_t total = export_bytes(m);
  *bytes = total;
  if (cap == 0) return UW_OK;
  if (!host_buf || cap < total) return UW_ERR_INVALID;
  if (!m->stream) return UW_ERR_STATE;
  UW_HIP(hipDeviceSynchronize());
  uint8_t* b = static_cast<uint8_t*>(host_buf);
  std::memset(b, 0, total);
  std::memcpy(b + kOffMagic, "UWF1", 4);
  wr32(b + kOffVersion, 1);
  wr32(b + kOffLayout, m->layout);
  wr32(b + kOffSegGroups, m->seg_groups);
  wr64(b + kOffRows, m->rows);
  wr64(b + kOffCols, m->cols);
  wr32(b + kOffPalSize, m->t.palette_size);
  wr32(b + kOffNCoded, m->t.n_coded);
  std::memcpy(b + kOffPalette, m->t.palette, 16);
  std::memcpy(b + kOffLen, m->t.code_len, 16);
  wr64(b + kOffV, m->V);
  wr64(b + kOffW, m->W);
  for (int v = 0; v < 256; ++v) wr64(b + kOffHist + 8 * v, m->t.hist[v]);
  for (int s = 0; s < kPal; ++s) wr64(b + kOffCoded + 8 * s, m->t.coded_count[s]);
  uint64_t at = kHeaderBytes;
  const void* src[6] = {m->sm, m->vflags, m->vrank, m->vexp, m->seg_off, m->stream};
  const uint64_t sz[6] = {m->numel, 4 * m->flag_words, 4 * m->flag_words, 64 * m->V, 4 * (m->segments + 1),
                          4 * (m->W + 2)};
  for (int i = 0; i < 6; ++i) {
    if (sz[i]) UW_HIP(hipMemcpy(b + at, src[i], sz[i], hipMemcpyDeviceToHost));
    at += pad256(sz[i]);
  }
  return UW_OK;
} catch (...) {
  return UW_ERR_NOMEM;
}

uw_status uw_import(const void* host_blob, size_t nbytes, void* stream, uw_matrix** out) try {
  if (!out) return UW_ERR_INVALID;
  *out = nullptr;
  if (!host_blob) return UW_ERR_INVALID;
  const uint8_t* b = static_cast<const uint8_t*>(host_blob);
  if (nbytes < kHeaderBytes || std::memcmp(b, "UWF1", 4) != 0) return UW_ERR_CORRUPT;
  if (rd32(b + kOffVersion) != 1) return UW_ERR_CORRUPT;
  const uint32_t layout = rd32(b + kOffLayout), sg = rd32(b + kOffSegGroups);
  const uint64_t rows = rd64(b + kOffRows), cols = rd64(b + kOffCols);
  if (layout > 1 || !valid_seg_groups(sg) || rows == 0 || cols == 0 || cols % kGroup != 0) return UW_ERR_CORRUPT;
  if (rows > (1ull << 32) || rows * cols >= (1ull << 32)) return UW_ERR_CORRUPT;

  uw_matrix tmp;
  shape_from(&tmp, rows, cols, layout, sg);
  tmp.V = rd64(b + kOffV);
  tmp.W = rd64(b + kOffW);
  if (tmp.V > tmp.groups || tmp.W >= (1ull << 32)) return UW_ERR_CORRUPT;
  for (int v = 0; v < 256; ++v) tmp.t.hist[v] = rd64(b + kOffHist + 8 * v);
  uint64_t hsum = 0;
  for (int v = 0; v < 256; ++v) hsum += tmp.t.hist[v];
  if (hsum != tmp.numel) return UW_ERR_CORRUPT;
  // the palette must be the one the histogram implies
  choose_palette(tmp.t);
  if (rd32(b + kOffPalSize) != tmp.t.palette_size || std::memcmp(b + kOffPalette, tmp.t.palette, 16) != 0)
    return UW_ERR_CORRUPT;
  uint64_t coded_sum = 0;
  for (int s = 0; s < kPal; ++s) {
    tmp.t.coded_count[s] = rd64(b + kOffCoded + 8 * s);
    if (tmp.t.coded_count[s] && (uint32_t)s >= tmp.t.palette_size) return UW_ERR_CORRUPT;
    coded_sum += tmp.t.coded_count[s];
  }
  if (coded_sum != (tmp.groups - tmp.V) * kGroup) return UW_ERR_CORRUPT;
  // the code must be the one the coded histogram implies
  finish_code(tmp.t);
  if (rd32(b + kOffNCoded) != tmp.t.n_coded || std::memcmp(b + kOffLen, tmp.t.code_len, 16) != 0)
    return UW_ERR_CORRUPT;
  if (export_bytes(&tmp) != nbytes) return UW_ERR_CORRUPT;

  // small sections: flags, ranks, offsets
  const uint64_t o_sm = kHeaderBytes, o_vf = o_sm + pad256(tmp.numel), o_vr = o_vf + pad256(4 * tmp.flag_words),
                 o_vx = o_vr + pad256(4 * tmp.flag_words), o_so = o_vx + pad256(64 * tmp.V),
                 o_st = o_so + pad256(4 * (tmp.segments + 1));
  std::vector<uint32_t> vf(tmp.flag_words), vr(tmp.flag_words), so(tmp.segments + 1);
  std::memcpy(vf.data(), b + o_vf, 4 * tmp.flag_words);
  std::memcpy(vr.data(), b + o_vr, 4 * tmp.flag_words);
  std::memcpy(so.data(), b + o_so, 4 * (tmp.segments + 1));
  uint64_t run = 0;
  for (uint64_t w = 0; w < tmp.flag_words; ++w) {
    if (vr[w] != run) return UW_ERR_CORRUPT;
    uint32_t f = vf[w];
    if (w == tmp.flag_words - 1 && (tmp.groups & 31)) f &= (1u << (tmp.groups & 31)) - 1u;
    if (f != vf[w]) return UW_ERR_CORRUPT;   // bits past the last group
    run += (uint64_t)__builtin_popcount(f);
  }
  if (run != tmp.V) return UW_ERR_CORRUPT;
  if (so[0] != 0 || so[tmp.segments] != tmp.W) return UW_ERR_CORRUPT;
  uint32_t maxlen = 0;
  for (int s = 0; s < kPal; ++s) maxlen = std::max<uint32_t>(maxlen, tmp.t.code_len[s]);
  for (uint64_t sgi = 0; sgi < tmp.segments; ++sgi) {
    if (so[sgi + 1] < so[sgi]) return UW_ERR_CORRUPT;
    uint64_t coded_groups = 0;
    const uint64_t g1 = std::min<uint64_t>((sgi + 1) * sg, tmp.groups);
    for (uint64_t g = sgi * sg; g < g1; ++g) coded_groups += ((vf[g >> 5] >> (g & 31)) & 1u) ? 0 : 1;
    const uint64_t words = so[sgi + 1] - so[sgi];
    if ((coded_groups == 0) != (words == 0)) return UW_ERR_CORRUPT;
    if (words > (coded_groups * kGroup * maxlen + 31) / 32) return UW_ERR_CORRUPT;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  uw_matrix* m = new (std::nothrow) uw_matrix();
  if (!m) return UW_ERR_NOMEM;
  struct Guard {
    uw_matrix* m;
    ~Guard() { if (m) { free_sections(m); delete m; } }
  } guard{m};
  UW_HIP(hipGetDevice(&m->device));
  m->alloc = current_allocator();
  shape_from(m, rows, cols, layout, sg);
  m->V = tmp.V;
  m->W = tmp.W;
  m->t = tmp.t;
  for (uint64_t w = 0; w * 64 < m->segments; ++w) {
    const uint64_t e = std::min<uint64_t>((w + 1) * 64, m->segments);
    m->wave_span = std::max<uint32_t>(m->wave_span, so[e] - (so[w * 64] & ~3u));
  }
  m->code_bits = 0;
  for (int i = 0; i < kPal; ++i) m->code_bits += m->t.coded_count[i] * m->t.code_len[i];
  const uint64_t sw = stream_alloc_words(m->W);
  UW_CHECK(dev_alloc(m->alloc, &m->sm, m->numel));
  UW_CHECK(dev_alloc(m->alloc, &m->vflags, 4 * m->flag_words));
  UW_CHECK(dev_alloc(m->alloc, &m->vrank, 4 * m->flag_words));
  UW_CHECK(dev_alloc(m->alloc, &m->vexp, 64 * m->V));
  UW_CHECK(dev_alloc(m->alloc, &m->seg_off, 4 * (m->segments + 1)));
  UW_CHECK(dev_alloc(m->alloc, &m->stream, 4 * sw));
  UW_CHECK(dev_alloc(m->alloc, &m->corrupt, sizeof(int)));
  UW_HIP(hipMemsetAsync(m->corrupt, 0, sizeof(int), s));
  UW_HIP(hipMemsetAsync(m->stream, 0, 4 * sw, s));
  UW_HIP(hipMemcpyAsync(m->sm, b + o_sm, m->numel, hipMemcpyHostToDevice, s));
  UW_HIP(hipMemcpyAsync(m->vflags, vf.data(), 4 * m->flag_words, hipMemcpyHostToDevice, s));
  UW_HIP(hipMemcpyAsync(m->vrank, vr.data(), 4 * m->flag_words, hipMemcpyHostToDevice, s));
  if (m->V) UW_HIP(hipMemcpyAsync(m->vexp, b + o_vx, 64 * m->V, hipMemcpyHostToDevice, s));
  UW_HIP(hipMemcpyAsync(m->seg_off, so.data(), 4 * (m->segments + 1), hipMemcpyHostToDevice, s));
  UW_HIP(hipMemcpyAsync(m->stream, b + o_st, 4 * (m->W + 2), hipMemcpyHostToDevice, s));
  UW_CHECK(upload_lut(m, s));   // synchronises
  guard.m = nullptr;
  *out = m;
  return UW_OK;
} catch (...) {
  return UW_ERR_NOMEM;
}

void uw_free(uw_matrix* m) {
  if (!m) return;
  free_sections(m);
  delete m;
}

static uw_status decode_to(const uw_matrix* m, void* out, int mode, hipStream_t s) {
  if (!m || !out || !aligned16(out)) return UW_ERR_INVALID;
  if (!m->stream) return UW_ERR_STATE;
  UW_HIP(launch_decode(decode_args(m, out), mode, s));
  return UW_OK;
}

uw_status uw_decode_full(const uw_matrix* m, uint16_t* w_out_dev, void* stream) {
  if (m && m->fp8) return UW_ERR_UNSUPPORTED;
  return decode_to(m, w_out_dev, kDecodeFull, static_cast<hipStream_t>(stream));
}

uw_status uw_decode_fp8(const uw_matrix* m, uint8_t* w_out_dev, void* stream) {
  if (m && !m->fp8) return UW_ERR_UNSUPPORTED;
  return decode_to(m, w_out_dev, kDecodeFp8, static_cast<hipStream_t>(stream));
}

uw_status uw_decode_exponent(const uw_matrix* m, uint8_t* e_out_dev, void* stream) {
  return decode_to(m, e_out_dev, kDecodeExponent, static_cast<hipStream_t>(stream));
}

uw_status uw_transcode_palette(uw_matrix* m, uint8_t* idx_out_dev, void* stream) {
  if (!m) return UW_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (idx_out_dev) return decode_to(m, idx_out_dev, kDecodeNibble, s);
  if (!m->stream) return m->pidx ? UW_OK : UW_ERR_STATE;
  if (!m->pidx) UW_CHECK(dev_alloc(m->alloc, &m->pidx, m->numel / 2));
  return decode_to(m, m->pidx, kDecodeNibble, s);
}

uw_status uw_drop_stream(uw_matrix* m, void* stream) {
  if (!m) return UW_ERR_INVALID;
  if (!m->pidx) return UW_ERR_STATE;
  UW_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  dev_free(m->alloc, m->stream);
  dev_free(m->alloc, m->seg_off);
  dev_free(m->alloc, m->lut);
  return UW_OK;
}

uw_status uw_drop_palette(uw_matrix* m, void* stream) {
  if (!m) return UW_ERR_INVALID;
  if (!m->stream) return UW_ERR_STATE;   // would leave no form to decode from
  UW_HIP(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  dev_free(m->alloc, m->pidx);
  return UW_OK;
}

uw_status uw_workspace_size(const uw_matrix* m, uw_pipeline p, int64_t batch, size_t* bytes) {
  if (!m || !bytes || batch <= 0 || !pipeline_arg(p)) return UW_ERR_INVALID;
  if (m->fp8) return UW_ERR_UNSUPPORTED;
  // enough for any kernel variant a cfg may select at this batch without a
  // forced split, and for the tuned choice
  const Plan r = plan_call(m, p, batch, nullptr);
  WeightView v = pipeline_view(m, r.p, nullptr);
  const size_t part = std::max(gemm_partial_elems_max(v, batch, 0), gemm_partial_elems(v, batch, r.cfgp()));
  *bytes = prep_bytes(m, r.p) + pad256(part * sizeof(float));
  return UW_OK;
}

uw_status uw_workspace_size_cfg(const uw_matrix* m, uw_pipeline p, int64_t batch, const uw_kernel_cfg* cfg,
                                size_t* bytes) {
  if (!m || !bytes || batch <= 0 || !pipeline_arg(p)) return UW_ERR_INVALID;
  if (m->fp8) return UW_ERR_UNSUPPORTED;
  const Plan r = plan_call(m, p, batch, cfg);
  *bytes = prep_bytes(m, r.p) + partial_bytes(m, r.p, batch, r.cfgp());
  return UW_OK;
}

static uw_status workspace_for(const uw_matrix* m, int p, int64_t batch, const uw_kernel_cfg* cfg, size_t* b) {
  *b = prep_bytes(m, p) + partial_bytes(m, p, batch, cfg);
  return UW_OK;
}

uw_status uw_matmul_reconstruct(const uw_matrix* m, uw_pipeline p, const uint16_t* x_dev, int64_t batch,
                                float* y_dev, void* ws_dev, size_t ws_bytes, const uw_kernel_cfg* cfg,
                                void* stream) {
  if (!m || !pipeline_arg(p) || batch <= 0) return UW_ERR_INVALID;
  if (m->fp8) return UW_ERR_UNSUPPORTED;
  const Plan r = plan_call(m, p, batch, cfg);
  UW_CHECK(check_matmul_args(m, r.p, x_dev, batch, y_dev));
  size_t need = 0;
  workspace_for(m, r.p, batch, r.cfgp(), &need);
  if (need > ws_bytes || (need && !ws_dev) || !aligned16(ws_dev)) return UW_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  UW_CHECK(preprocess(m, r.p, ws, s));
  WeightView v = pipeline_view(m, r.p, ws);
  const size_t pb = prep_bytes(m, r.p);
  float* part = reinterpret_cast<float*>(ws + pb);
  UW_HIP(launch_gemm(v, x_dev, batch, y_dev, (int64_t)v.n, 0, r.cfgp(), part, (need - pb) / sizeof(float), s));
  return UW_OK;
}

uw_status uw_matmul_stage(const uw_matrix* m, uw_pipeline p, const void* prep_dev, const uint16_t* x_dev,
                          int64_t batch, float* y_dev, void* ws_dev, size_t ws_bytes, const uw_kernel_cfg* cfg,
                          void* stream) {
  size_t need = 0;
  return uw::matmul_stage_into(m, p, prep_dev, x_dev, batch, y_dev, ws_dev, ws_bytes, cfg,
                               static_cast<hipStream_t>(stream), &need);
}

}  // extern "C"

uw_status uw::matmul_stage_into(const uw_matrix* m, int p, const void* prep_dev, const uint16_t* x_dev,
                                int64_t batch, float* y_dev, void* part, size_t part_bytes,
                                const uw_kernel_cfg* cfg, hipStream_t s, size_t* need_out) {
  *need_out = 0;
  if (!m || !x_dev || !y_dev || batch <= 0 || p < UW_PIPE_FULL || p > UW_PIPE_PALETTE_DIRECT) return UW_ERR_INVALID;
  if (m->fp8) return UW_ERR_UNSUPPORTED;
  if (!aligned16(x_dev) || (reinterpret_cast<uintptr_t>(y_dev) & 3u)) return UW_ERR_INVALID;
  if (logical_k(m) % 8 != 0) return UW_ERR_UNSUPPORTED;
  if (p == UW_PIPE_PALETTE_DIRECT) {
    if (!m->pidx) return UW_ERR_STATE;
  } else if (!prep_dev || !aligned16(prep_dev)) {
    return UW_ERR_INVALID;
  }
  const Plan r = plan_call(m, p, batch, cfg);
  const size_t need = partial_bytes(m, p, batch, r.cfgp());
  *need_out = need;
  if (need > part_bytes || (need && !part) || !aligned16(part)) return UW_ERR_WORKSPACE;
  WeightView v = pipeline_view(m, p, prep_dev);
  UW_HIP(launch_gemm(v, x_dev, batch, y_dev, (int64_t)v.n, 0, r.cfgp(), static_cast<float*>(part),
                     need / sizeof(float), s));
  return UW_OK;
}

extern "C" {

}  // extern "C"

namespace {

// Workspace of a grouped call: the per-matrix layout (each matrix's
// preprocessed form and partial sums back to back), or when the group runs
// as one LDS-tiled launch, the preprocessed forms packed and the group's
// partial rows after them; the larger of the two, so the one-launch form is
// always available.  *tile_part = partial floats of that launch (SIZE_MAX:
// the group does not run as one).
uw_status grouped_need(const uw_matrix* const* ms, int count, int p, int64_t batch, const uw_kernel_cfg* cfg,
                       size_t* need, size_t* prep_total, size_t* tile_part) {
  size_t per = 0, prep = 0;
  for (int i = 0; i < count; ++i) {
    size_t b = 0;
    workspace_for(ms[i], p, batch, cfg, &b);
    per += b;
    prep += prep_bytes(ms[i], p);
  }
  size_t tp = SIZE_MAX;
  if (count >= 2 && count <= kGroupMax) {
    WeightView plan[kGroupMax];
    for (int i = 0; i < count; ++i) plan[i] = pipeline_view(ms[i], p, nullptr);
    tp = gemm_tile_group_partial_elems(plan, count, batch, cfg);
  }
  *need = tp == SIZE_MAX ? per : std::max(per, (size_t)pad256(prep) + tp * sizeof(float));
  *prep_total = prep;
  *tile_part = tp;
  return UW_OK;
}

uw_status check_group_args(const uw_matrix* const* ms, int count, int p, const uint16_t* x_dev, int64_t batch,
                           const float* y_dev) {
  if (!ms || count <= 0) return UW_ERR_INVALID;
  for (int i = 0; i < count; ++i) {
    UW_CHECK(check_matmul_args(ms[i], p, x_dev, batch, y_dev));
    if (logical_k(ms[i]) != logical_k(ms[0])) return UW_ERR_INVALID;
  }
  return UW_OK;
}

}  // namespace

extern "C" {

uw_status uw_workspace_size_grouped(const uw_matrix* const* ms, int count, uw_pipeline p, int64_t batch,
                                    const uw_kernel_cfg* cfg, size_t* bytes) {
  if (!ms || count <= 0 || !bytes || batch <= 0 || !pipeline_arg(p)) return UW_ERR_INVALID;
  for (int i = 0; i < count; ++i) {
    if (!ms[i]) return UW_ERR_INVALID;
    if (ms[i]->fp8) return UW_ERR_UNSUPPORTED;
  }
  const Plan gp = plan_group(ms, count, p, batch, cfg);
  size_t prep = 0, tp = 0;
  return grouped_need(ms, count, gp.p, batch, gp.cfgp(), bytes, &prep, &tp);
}

uw_status uw_matmul_reconstruct_grouped(const uw_matrix* const* ms, int count, uw_pipeline p,
                                        const uint16_t* x_dev, int64_t batch, float* y_dev, void* ws_dev,
                                        size_t ws_bytes, const uw_kernel_cfg* cfg_in, void* stream) {
  if (!ms || count <= 0 || !pipeline_arg(p) || batch <= 0) return UW_ERR_INVALID;
  for (int i = 0; i < count; ++i) {
    if (!ms[i]) return UW_ERR_INVALID;
    if (ms[i]->fp8) return UW_ERR_UNSUPPORTED;
  }
  const Plan gp = plan_group(ms, count, p, batch, cfg_in);
  const int rp = gp.p;
  const uw_kernel_cfg* cfg = gp.cfgp();
  UW_CHECK(check_group_args(ms, count, rp, x_dev, batch, y_dev));
  uint64_t total_n = 0;
  for (int i = 0; i < count; ++i) total_n += logical_n(ms[i]);
  // the smallest workspace that runs the matrices one by one
  size_t need_per = 0;
  for (int i = 0; i < count; ++i) {
    size_t b = 0;
    workspace_for(ms[i], rp, batch, cfg, &b);
    need_per += b;
  }
  if (need_per > ws_bytes || (need_per && !ws_dev) || !aligned16(ws_dev)) return UW_ERR_WORKSPACE;
  size_t need_all = 0, prep_total = 0, tile_part = SIZE_MAX;
  UW_CHECK(grouped_need(ms, count, rp, batch, cfg, &need_all, &prep_total, &tile_part));
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  // Matrices whose kernel (as one matrix as wide as the group) is an LDS tile
  // share one launch: fixed per-launch costs are paid once and K is split for
  // the group's tiles together.  Its workspace: the preprocessed weights
  // packed first, the group's partial rows after them.
  const size_t part_off = pad256(prep_total);
  const bool tile_group = tile_part != SIZE_MAX && part_off + tile_part * sizeof(float) <= ws_bytes;
  size_t off = 0;
  std::vector<size_t> offs((size_t)count);
  for (int i = 0; i < count; ++i) {
    offs[(size_t)i] = off;
    UW_CHECK(preprocess(ms[i], rp, ws + off, s));
    size_t b = prep_bytes(ms[i], rp);
    if (!tile_group) workspace_for(ms[i], rp, batch, cfg, &b);
    off += b;
  }
  if (count >= 2 && count <= kGroupMax) {
    WeightView vs[kGroupMax];
    int64_t c0[kGroupMax];
    int64_t col = 0;
    for (int i = 0; i < count; ++i) {
      vs[i] = pipeline_view(ms[i], rp, ws + offs[(size_t)i]);
      c0[i] = col;
      col += (int64_t)vs[i].n;
    }
    // matrices that all run the VALU GEMV share one launch
    const hipError_t e = launch_gemm_group(vs, count, x_dev, batch, y_dev, (int64_t)total_n, c0, cfg, s);
    if (e == hipSuccess) return UW_OK;
    if (e != hipErrorNotSupported) return UW_ERR_DEVICE;
    if (tile_group) {
      float* part = tile_part ? reinterpret_cast<float*>(ws + part_off) : nullptr;
      UW_HIP(launch_gemm_tile_group(vs, count, x_dev, batch, y_dev, (int64_t)total_n, c0, cfg, part, tile_part, s));
      return UW_OK;
    }
  }
  uint64_t col0 = 0;
  for (int i = 0; i < count; ++i) {
    WeightView v = pipeline_view(ms[i], rp, ws + offs[(size_t)i]);
    const size_t pb = prep_bytes(ms[i], rp);
    size_t b = 0;
    workspace_for(ms[i], rp, batch, cfg, &b);
    float* part = reinterpret_cast<float*>(ws + offs[(size_t)i] + pb);
    UW_HIP(launch_gemm(v, x_dev, batch, y_dev, (int64_t)total_n, (int64_t)col0, cfg, part,
                       (b - pb) / sizeof(float), s));
    col0 += v.n;
  }
  return UW_OK;
}

uw_status uw_gemm_bf16(const uint16_t* w_dev, int64_t n, int64_t k, uw_layout layout, const uint16_t* x_dev,
                       int64_t batch, float* y_dev, const uw_kernel_cfg* cfg, void* stream) {
  if (!w_dev || !x_dev || !y_dev || n <= 0 || k <= 0 || batch <= 0) return UW_ERR_INVALID;
  if (layout != UW_LAYOUT_NK && layout != UW_LAYOUT_KN) return UW_ERR_INVALID;
  if (!aligned16(w_dev) || !aligned16(x_dev)) return UW_ERR_INVALID;
  const uint64_t cols = layout == UW_LAYOUT_NK ? (uint64_t)k : (uint64_t)n;
  if (cols % 64 != 0 || k % 8 != 0) return UW_ERR_UNSUPPORTED;
  WeightView v;
  std::memset(&v, 0, sizeof(v));
  v.fmt = kFmtBf16;
  v.layout = (int)layout;
  v.n = (uint64_t)n;
  v.k = (uint64_t)k;
  v.bf16 = w_dev;
  const size_t pe = gemm_partial_elems(v, batch, cfg);
  float* part = nullptr;
  const uw_allocator alloc = current_allocator();
  if (pe) UW_CHECK(dev_alloc(alloc, &part, pe * sizeof(float)));   // yardstick path only
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_gemm(v, x_dev, batch, y_dev, n, 0, cfg, part, pe, s);
  if (part) {
    (void)hipStreamSynchronize(s);
    dev_free(alloc, part);
  }
  return e == hipSuccess ? UW_OK : UW_ERR_DEVICE;
}

int32_t uw_variant_count(void) { return gemm_variant_count(); }

uw_status uw_plan_gemm(const uw_matrix* m, uw_pipeline p, int64_t batch, const uw_kernel_cfg* cfg,
                       uw_gemm_plan* out) {
  if (!m || !out || batch <= 0 || !pipeline_arg(p)) return UW_ERR_INVALID;
  if (m->fp8) return UW_ERR_UNSUPPORTED;
  std::memset(out, 0, sizeof(*out));
  const Plan r = plan_call(m, p, batch, cfg);
  if (!pipeline_feasible(m, r.p)) return UW_ERR_STATE;
  out->pipeline = r.p;
  describe_gemm(pipeline_view(m, r.p, nullptr), batch, r.cfgp(), out);
  return UW_OK;
}

}  // extern "C"

namespace {

// Jobs with UW_PIPE_AUTO resolved and empty cfgs replaced by the tuned choice.
uw_status resolve_jobs(const uw_job* jobs, int count, std::vector<uw_job>& out) {
  if (!jobs || count <= 0) return UW_ERR_INVALID;
  out.assign(jobs, jobs + count);
  for (int i = 0; i < count; ++i) {
    uw_job& j = out[(size_t)i];
    if (!j.m || !pipeline_arg(j.pipeline) || j.batch <= 0) return UW_ERR_INVALID;
    if (j.m->fp8) return UW_ERR_UNSUPPORTED;
    const Plan r = plan_call(j.m, j.pipeline, j.batch, cfg_empty(j.cfg) ? nullptr : &j.cfg);
    j.pipeline = r.p;
    if (r.has_cfg) j.cfg = r.cfg;
  }
  return UW_OK;
}

uw_status sequence_need(const std::vector<uw_job>& jobs, size_t* prep_out, size_t* bytes) {
  size_t prep = 0, part = 0;
  for (const uw_job& j : jobs) {
    prep = std::max(prep, prep_bytes(j.m, j.pipeline));
    part = std::max(part, partial_bytes(j.m, j.pipeline, j.batch, &j.cfg));
  }
  *prep_out = prep;
  *bytes = 2 * prep + part;
  return UW_OK;
}

}  // namespace

extern "C" {

uw_status uw_sequence_workspace_size(const uw_job* jobs, int count, size_t* bytes) try {
  if (!jobs || count <= 0 || !bytes) return UW_ERR_INVALID;
  std::vector<uw_job> rj;
  UW_CHECK(resolve_jobs(jobs, count, rj));
  size_t prep = 0;
  return sequence_need(rj, &prep, bytes);
} catch (...) {
  return UW_ERR_NOMEM;
}

uw_status uw_run_sequence(const uw_job* jobs_in, int count, int32_t decode_cus, void* ws_dev, size_t ws_bytes,
                          void* stream) try {
  if (!jobs_in || count <= 0) return UW_ERR_INVALID;
  std::vector<uw_job> rj;
  UW_CHECK(resolve_jobs(jobs_in, count, rj));
  return uw::run_jobs(rj.data(), count, decode_cus, ws_dev, ws_bytes, static_cast<hipStream_t>(stream));
} catch (...) {
  return UW_ERR_NOMEM;
}

}  // extern "C"

// Jobs as given: explicit pipelines, each cfg used as it is (fields <= 0 are
// the library defaults).  The autotuner times candidates through this, so
// the tuning table never stands in for a candidate.
uw_status uw::jobs_workspace(const uw_job* jobs, int count, size_t* bytes) try {
  if (!jobs || count <= 0 || !bytes) return UW_ERR_INVALID;
  for (int i = 0; i < count; ++i)
    if (!jobs[i].m || jobs[i].pipeline < UW_PIPE_FULL || jobs[i].pipeline > UW_PIPE_PALETTE_DIRECT)
      return UW_ERR_INVALID;
  std::vector<uw_job> v(jobs, jobs + count);
  size_t prep = 0;
  return sequence_need(v, &prep, bytes);
} catch (...) {
  return UW_ERR_NOMEM;
}

uw_status uw::run_jobs(const uw_job* jobs, int count, int32_t decode_cus, void* ws_dev, size_t ws_bytes,
                       hipStream_t s) try {
  if (!jobs || count <= 0) return UW_ERR_INVALID;
  std::vector<uw_job> rj(jobs, jobs + count);
  for (int i = 0; i < count; ++i)
    UW_CHECK(check_matmul_args(jobs[i].m, jobs[i].pipeline, jobs[i].x_dev, jobs[i].batch, jobs[i].y_dev));
  size_t need = 0, prep = 0;
  UW_CHECK(sequence_need(rj, &prep, &need));
  if (need > ws_bytes || (need && !ws_dev) || !aligned16(ws_dev)) return UW_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  uint8_t* bufs[2] = {ws, ws + prep};
  float* part = reinterpret_cast<float*>(ws + 2 * prep);
  const size_t part_elems = (need - 2 * prep) / sizeof(float);

  bool any_split = false;
  for (int i = 0; i < count; ++i) {
    const int d = jobs[i].cfg.decode_cus > 0 ? jobs[i].cfg.decode_cus : decode_cus;
    if (d > 0 && jobs[i].pipeline != UW_PIPE_PALETTE_DIRECT) any_split = true;
  }
  if (!any_split) {   // everything in order on the caller's stream
    for (int i = 0; i < count; ++i) {
      const uw_job& j = jobs[i];
      UW_CHECK(preprocess(j.m, j.pipeline, bufs[0], s));
      WeightView v = pipeline_view(j.m, j.pipeline, bufs[0]);
      UW_HIP(launch_gemm(v, j.x_dev, j.batch, j.y_dev, (int64_t)v.n, 0, &j.cfg, part, part_elems, s));
    }
    return UW_OK;
  }

  // Per job: its preprocessing runs on a stream masked to D CUs and its GEMM on
  // a stream masked to the other CUs (D = the job's decode_cus, else the
  // sequence default; D = 0 puts both on the caller's stream).  GEMMs stay in
  // job order; preprocessing of job i waits for the GEMM of job i-2, which
  // used the same buffer.  The streams and events belong to the library
  // (runtime.cpp); one sequence runs at a time.
  std::lock_guard<std::mutex> seq(sequence_mutex());
  hipEvent_t* pool = nullptr;
  UW_CHECK(pooled_events(2 * (size_t)count + 1, &pool));
  hipEvent_t fork = pool[0];
  hipEvent_t* prep_done = pool + 1;
  hipEvent_t* gemm_done = pool + 1 + count;
  UW_HIP(hipEventRecord(fork, s));
  std::vector<hipStream_t> used;
  auto enter = [&](hipStream_t st) -> uw_status {
    if (st == s) return UW_OK;
    for (hipStream_t u : used)
      if (u == st) return UW_OK;
    UW_HIP(hipStreamWaitEvent(st, fork, 0));
    used.push_back(st);
    return UW_OK;
  };
  for (int i = 0; i < count; ++i) {
    const uw_job& j = jobs[i];
    const int d = j.cfg.decode_cus > 0 ? j.cfg.decode_cus : decode_cus;
    hipStream_t ds = s, gs = s;
    if (d > 0 && j.pipeline != UW_PIPE_PALETTE_DIRECT) {
      SplitStreams ss;
      UW_CHECK(split_streams(d, &ss));
      ds = ss.dec;
      gs = ss.gemm;
    }
    UW_CHECK(enter(ds));
    UW_CHECK(enter(gs));
    uint8_t* buf = bufs[i & 1];
    if (j.pipeline != UW_PIPE_PALETTE_DIRECT) {
      if (i >= 2) UW_HIP(hipStreamWaitEvent(ds, gemm_done[i - 2], 0));
      UW_CHECK(preprocess(j.m, j.pipeline, buf, ds));
      UW_HIP(hipEventRecord(prep_done[i], ds));
      UW_HIP(hipStreamWaitEvent(gs, prep_done[i], 0));
    }
    if (i >= 1) UW_HIP(hipStreamWaitEvent(gs, gemm_done[i - 1], 0));
    WeightView v = pipeline_view(j.m, j.pipeline, buf);
    UW_HIP(launch_gemm(v, j.x_dev, j.batch, j.y_dev, (int64_t)v.n, 0, &j.cfg, part, part_elems, gs));
    UW_HIP(hipEventRecord(gemm_done[i], gs));
  }
  // join: the last GEMM follows every earlier GEMM and preprocessing it needed;
  // make the caller's stream wait for it and for any preprocessing stream
  UW_HIP(hipStreamWaitEvent(s, gemm_done[count - 1], 0));
  for (hipStream_t u : used) {
    UW_HIP(hipEventRecord(prep_done[0], u));
    UW_HIP(hipStreamWaitEvent(s, prep_done[0], 0));
  }
  return UW_OK;
} catch (...) {
  return UW_ERR_NOMEM;
}

extern "C" {

uw_status uw_sync_status(const uw_matrix* m, void* stream) {
  if (!m) return UW_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  UW_HIP(hipStreamSynchronize(s));
  int flag = 0;
  UW_HIP(hipMemcpy(&flag, m->corrupt, sizeof(int), hipMemcpyDeviceToHost));
  if (flag) {
    UW_HIP(hipMemset(m->corrupt, 0, sizeof(int)));
    return UW_ERR_CORRUPT;
  }
  return UW_OK;
}

}  // extern "C"
