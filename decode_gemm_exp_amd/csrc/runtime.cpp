// runtime.cpp -- process-wide state of libunweight:
//   * the device allocator every section and scratch buffer comes from
//     (uw_set_allocator; hipMalloc / hipFree by default);
//   * the HIP objects the sequence runner keeps between calls (one pair of
//     CU-masked streams per device and CU share, one event pool per device)
//     and their owner: uw_release_resources destroys them, and an exit
//     handler registered when the first of them is created does the same
//     before the HIP runtime's own teardown;
//   * the table of tuned choices (uw_set_tuning, uw_load_tuning) that pipeline
//     UW_PIPE_AUTO and a NULL kernel configuration consult.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "自動調優機制": the tuner's
// product is a per-model configuration that fixes, per projection and batch
// size, the pipeline, the matmul variant and the compute split; at run time the
// engine looks the choice up instead of deciding again.
#include <hip/hip_ext.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "uw_internal.h"

namespace uw {
namespace {

// ---- allocator --------------------------------------------------------------------
std::mutex g_alloc_mu;
uw_allocator g_alloc{};   // alloc == NULL: hipMalloc / hipFree

// ---- sequence-runner HIP objects -----------------------------------------------------
std::mutex g_res_mu;
std::map<std::pair<int, int>, SplitStreams> g_split;   // (device, decode CUs)
std::map<int, std::vector<hipEvent_t>> g_events;      // per device
std::mutex g_seq_mu;                                   // one sequence at a time per process
bool g_exit_hook = false;

// Destroy every stream and event the library created.  Each object belongs to
// the device it was created on, which is made current for the call.
void release_locked(bool sync) {
  int cur = -1;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_split) {
    if (hipSetDevice(kv.first.first) != hipSuccess) continue;
    for (hipStream_t st : {kv.second.dec, kv.second.gemm}) {
      if (!st) continue;
      if (sync) (void)hipStreamSynchronize(st);
      (void)hipStreamDestroy(st);
    }
  }
  g_split.clear();
  for (auto& kv : g_events) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    for (hipEvent_t e : kv.second) (void)hipEventDestroy(e);
  }
  g_events.clear();
  if (cur >= 0) (void)hipSetDevice(cur);
}

// Runs at exit() before the HIP runtime's static destructors: it is
// registered after the runtime was initialised, and exit handlers run in the
// reverse order of registration.
void release_at_exit() {
  std::lock_guard<std::mutex> lk(g_res_mu);
  release_locked(false);
}

void need_exit_hook() {   // g_res_mu held
  if (!g_exit_hook) {
    g_exit_hook = true;
    std::atexit(release_at_exit);
  }
}

std::vector<uint32_t> cu_mask(int total, int first, int count) {
  std::vector<uint32_t> m((size_t)(total + 31) / 32, 0u);
  for (int i = first; i < first + count && i < total; ++i) m[(size_t)i / 32] |= 1u << (i % 32);
  return m;
}

// ---- tuned choices ---------------------------------------------------------------------
using TuneKey = std::tuple<uint64_t, uint64_t, int32_t, int32_t, int32_t>;   // n, k, layout, residency, group
std::mutex g_tune_mu;
std::map<TuneKey, std::vector<uw_tune_entry>> g_tune;

bool entry_valid(const uw_tune_entry& e) {
  return e.batch > 0 && e.n > 0 && e.k > 0 && (e.layout == 0 || e.layout == 1) && e.residency >= 1 &&
         e.residency <= 3 && e.pipeline >= UW_PIPE_FULL && e.pipeline <= UW_PIPE_PALETTE_DIRECT &&
         e.variant >= 0 && e.variant <= gemm_variant_count() && e.split_k >= 0 && e.decode_cus >= 0 &&
         (e.group == 0 || (e.group >= 2 && e.group <= kTuneGroupMax)) &&
         gemm_variant_supported(e.variant <= 0 ? 1 : e.variant, e.layout);
}

void add_locked(const uw_tune_entry& e) {
  auto& v = g_tune[TuneKey{e.n, e.k, e.layout, e.residency, e.group}];
  for (auto& old : v)
    if (old.batch == e.batch) {
      old = e;
      return;
    }
  v.push_back(e);
}

// Integer value of "key": in one JSON object's text; false when absent.
bool json_int(const std::string& obj, const char* key, long long* out) {
  const std::string pat = std::string("\"") + key + "\"";
  size_t at = obj.find(pat);
  if (at == std::string::npos) return false;
  at = obj.find(':', at + pat.size());
  if (at == std::string::npos) return false;
  const char* p = obj.c_str() + at + 1;
  char* end = nullptr;
  const long long v = std::strtoll(p, &end, 10);
  if (end == p) return false;
  *out = v;
  return true;
}

bool json_double(const std::string& obj, const char* key, double* out) {
  const std::string pat = std::string("\"") + key + "\"";
  size_t at = obj.find(pat);
  if (at == std::string::npos) return false;
  at = obj.find(':', at + pat.size());
  if (at == std::string::npos) return false;
  const char* p = obj.c_str() + at + 1;
  char* end = nullptr;
  const double v = std::strtod(p, &end);
  if (end == p) return false;
  *out = v;
  return true;
}

}  // namespace

// ---- interfaces used by the rest of the library -----------------------------------

uw_allocator current_allocator() {
  std::lock_guard<std::mutex> lk(g_alloc_mu);
  return g_alloc;
}

uw_status alloc_with(const uw_allocator& a, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return UW_OK;
  if (a.alloc) {
    void* q = a.alloc(bytes, a.ctx);
    if (!q) return UW_ERR_NOMEM;
    if ((reinterpret_cast<uintptr_t>(q) & 255u) != 0) {   // sections are read with aligned vector loads
      if (a.free) a.free(q, a.ctx);
      return UW_ERR_INVALID;
    }
    *p = q;
    return UW_OK;
  }
  const hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return e == hipErrorOutOfMemory ? UW_ERR_NOMEM : UW_ERR_DEVICE;
  }
  return UW_OK;
}

void free_with(const uw_allocator& a, void* p) {
  if (!p) return;
  if (a.alloc) {
    if (a.free) a.free(p, a.ctx);
  } else {
    (void)hipFree(p);
  }
}

uw_status split_streams(int decode_cus, SplitStreams* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return UW_ERR_DEVICE;
  int total = 0;
  if (hipDeviceGetAttribute(&total, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || total <= 0)
    return UW_ERR_DEVICE;
  if (decode_cus <= 0) return UW_ERR_INVALID;
  if (decode_cus > total) decode_cus = total;
  std::lock_guard<std::mutex> lk(g_res_mu);
  auto it = g_split.find({dev, decode_cus});
  if (it != g_split.end()) {
    *out = it->second;
    return UW_OK;
  }
  need_exit_hook();
  SplitStreams ss;
  hipError_t e1, e2;
  if (decode_cus >= total) {
    // no mask: the two kernels share every CU, the hardware interleaves their blocks
    e1 = hipStreamCreateWithFlags(&ss.dec, hipStreamNonBlocking);
    e2 = e1 == hipSuccess ? hipStreamCreateWithFlags(&ss.gemm, hipStreamNonBlocking) : e1;
  } else {
    const std::vector<uint32_t> md = cu_mask(total, 0, decode_cus);
    const std::vector<uint32_t> mg = cu_mask(total, decode_cus, total - decode_cus);
    e1 = hipExtStreamCreateWithCUMask(&ss.dec, (uint32_t)md.size(), md.data());
    e2 = e1 == hipSuccess ? hipExtStreamCreateWithCUMask(&ss.gemm, (uint32_t)mg.size(), mg.data()) : e1;
  }
  if (e1 != hipSuccess || e2 != hipSuccess) {
    if (ss.dec) (void)hipStreamDestroy(ss.dec);
    if (ss.gemm) (void)hipStreamDestroy(ss.gemm);
    return UW_ERR_DEVICE;
  }
  g_split[{dev, decode_cus}] = ss;
  *out = ss;
  return UW_OK;
}

std::mutex& sequence_mutex() { return g_seq_mu; }

uw_status pooled_events(size_t count, hipEvent_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return UW_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_res_mu);
  need_exit_hook();
  std::vector<hipEvent_t>& pool = g_events[dev];
  while (pool.size() < count) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return UW_ERR_DEVICE;
    pool.push_back(e);
  }
  *out = pool.data();   // stable until the pool grows: callers hold sequence_mutex()
  return UW_OK;
}

int residency_of(const uw_matrix* m) { return (m->stream ? 1 : 0) | (m->pidx ? 2 : 0); }

// ---- timing aid (uw_set_kernel_events) -------------------------------------------------
std::atomic<void*> g_kev_before{nullptr}, g_kev_after{nullptr};

void kernel_event_before(hipStream_t s) {
  if (void* e = g_kev_before.load(std::memory_order_relaxed)) (void)hipEventRecord(static_cast<hipEvent_t>(e), s);
}
void kernel_event_after(hipStream_t s) {
  if (void* e = g_kev_after.load(std::memory_order_relaxed)) (void)hipEventRecord(static_cast<hipEvent_t>(e), s);
}

bool tuned_lookup(uint64_t n, uint64_t k, int layout, int residency, int64_t batch, uw_tune_entry* out,
                  int group) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto it = g_tune.find(TuneKey{n, k, layout, residency, group});
  if (it == g_tune.end() || it->second.empty() || batch <= 0) return false;
  // the tuned batch nearest on a log scale; ties go to the smaller batch
  const double lb = std::log2((double)batch);
  const uw_tune_entry* best = nullptr;
  double bd = 0;
  for (const uw_tune_entry& e : it->second) {
    const double d = std::fabs(std::log2((double)e.batch) - lb);
    if (!best || d < bd - 1e-12 || (std::fabs(d - bd) <= 1e-12 && e.batch < best->batch)) {
      best = &e;
      bd = d;
    }
  }
  *out = *best;
  return true;
}

}  // namespace uw

using namespace uw;

extern "C" {

uw_status uw_set_allocator(const uw_allocator* a) {
  if (a && ((a->alloc == nullptr) != (a->free == nullptr))) return UW_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_alloc_mu);
  if (a && a->alloc) {
    g_alloc = *a;
  } else {
    std::memset(&g_alloc, 0, sizeof(g_alloc));
  }
  return UW_OK;
}

uw_status uw_set_kernel_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return UW_ERR_INVALID;
  g_kev_before.store(before, std::memory_order_relaxed);
  g_kev_after.store(after, std::memory_order_relaxed);
  return UW_OK;
}

uw_status uw_release_resources(void) {
  std::lock_guard<std::mutex> seq(g_seq_mu);
  std::lock_guard<std::mutex> lk(g_res_mu);
  release_locked(true);
  return UW_OK;
}

uw_status uw_set_tuning(const uw_tune_entry* entries, int count) {
  if (count < 0 || (count > 0 && !entries)) return UW_ERR_INVALID;
  for (int i = 0; i < count; ++i)
    if (!entry_valid(entries[i])) return UW_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (int i = 0; i < count; ++i) add_locked(entries[i]);
  return UW_OK;
}

uw_status uw_clear_tuning(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune.clear();
  return UW_OK;
}

uw_status uw_load_tuning(const char* json_path) try {
  if (!json_path) return UW_ERR_INVALID;
  FILE* f = std::fopen(json_path, "rb");
  if (!f) return UW_ERR_INVALID;
  std::string text;
  char buf[4096];
  size_t got;
  while ((got = std::fread(buf, 1, sizeof(buf), f)) > 0) text.append(buf, got);
  std::fclose(f);
  const size_t list = text.find("\"entries\"");
  if (list == std::string::npos) return UW_ERR_CORRUPT;
  size_t at = text.find('[', list);
  if (at == std::string::npos) return UW_ERR_CORRUPT;
  const size_t list_end = text.find(']', at);
  if (list_end == std::string::npos) return UW_ERR_CORRUPT;
  std::vector<uw_tune_entry> got_entries;
  while (true) {
    const size_t o = text.find('{', at);
    if (o == std::string::npos || o > list_end) break;
    const size_t c = text.find('}', o);
    if (c == std::string::npos || c > list_end) return UW_ERR_CORRUPT;
    const std::string obj = text.substr(o, c - o + 1);
    long long v[10];
    static const char* keys[10] = {"batch", "projection", "n", "k", "layout", "residency",
                                   "pipeline", "variant", "split_k", "decode_cus"};
    for (int i = 0; i < 10; ++i)
      if (!json_int(obj, keys[i], &v[i])) return UW_ERR_CORRUPT;
    uw_tune_entry e;
    std::memset(&e, 0, sizeof(e));
    e.batch = v[0];
    e.projection = (int32_t)v[1];
    e.n = v[2] > 0 ? (uint64_t)v[2] : 0;
    e.k = v[3] > 0 ? (uint64_t)v[3] : 0;
    e.layout = (int32_t)v[4];
    e.residency = (int32_t)v[5];
    e.pipeline = (int32_t)v[6];
    e.variant = (int32_t)v[7];
    e.split_k = (int32_t)v[8];
    e.decode_cus = (int32_t)v[9];
    long long g = 0;
    if (json_int(obj, "group", &g)) {   // absent: an entry for calls on one matrix
      if (g < 0 || g > kTuneGroupMax) return UW_ERR_CORRUPT;
      e.group = (int32_t)g;
    }
    double us = 0;
    if (json_double(obj, "sequence_us", &us)) e.sequence_us = us;
    if (!entry_valid(e)) return UW_ERR_CORRUPT;
    got_entries.push_back(e);
    at = c + 1;
  }
  std::lock_guard<std::mutex> lk(g_tune_mu);
  for (const uw_tune_entry& e : got_entries) add_locked(e);
  return UW_OK;
} catch (...) {
  return UW_ERR_NOMEM;
}

uw_status uw_lookup_tuning(uint64_t n, uint64_t k, int32_t layout, int32_t residency, int64_t batch,
                           uw_tune_entry* out) {
  if (!out || batch <= 0 || (layout != 0 && layout != 1) || residency < 1 || residency > 3) return UW_ERR_INVALID;
  return tuned_lookup(n, k, layout, residency, batch, out) ? UW_OK : UW_ERR_STATE;
}

uw_status uw_lookup_tuning_grouped(uint64_t n, uint64_t k, int32_t layout, int32_t residency, int32_t group,
                                   int64_t batch, uw_tune_entry* out) {
  if (!out || batch <= 0 || (layout != 0 && layout != 1) || residency < 1 || residency > 3 || group < 2 ||
      group > kTuneGroupMax)
    return UW_ERR_INVALID;
  return tuned_lookup(n, k, layout, residency, batch, out, group) ? UW_OK : UW_ERR_STATE;
}

}  // extern "C"
