// autotune.cpp -- per-projection, per-batch choice of pipeline, GEMM variant
// and CU split, by measurement.
//
// [EVC] = "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
// (easyvibecoding.app/curated/736).  Section "自動調優機制" (autotuning): the
// tuner measures real end-to-end throughput on the target hardware, sweeps
// the gate projection with up and down fixed, then up, then down, and repeats
// until nothing improves; the result is a per-model configuration giving, per
// projection and batch size, the pipeline, the matmul variant and the compute
// split.  Section "解壓與運算資源共享": that split is a tunable found by
// measurement.  Section "四種執行管道": no pipeline wins everywhere.
//
// Objective: wall time (HIP events) of one pass over every given matrix in
// order, run by uw_run_sequence with the candidate configuration, median of
// three runs after a warm-up, with activations drawn from N(0,1) in BF16 (the
// matrix cores' power, and so the clock they hold, depends on the operand
// values; all-zero activations would tune for a faster chip than the one that
// runs).  Candidates per projection: every pipeline all its matrices can run
// (direct palette needs resident indices, the others the Huffman stream) x
// every GEMM variant that suits the batch; then the K split of the chosen
// kernel; then, for a pipeline with preprocessing, the CUs given to the
// preprocessing kernel.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "uw_internal.h"

namespace {

struct Choice {
  int32_t pipeline = UW_PIPE_EXPONENT, variant = 0, split_k = 0, decode_cus = 0;
  bool operator==(const Choice& o) const {
    return pipeline == o.pipeline && variant == o.variant && split_k == o.split_k && decode_cus == o.decode_cus;
  }
};

// Device buffers and HIP objects of one tuning run, released on every return.
// A return in the middle of a timed pass may leave launches that use x, y and
// the workspace in flight, so the stream is drained before they are freed (an
// allocator hook may hand them out again at once).
struct Bufs {
  uw_allocator a = uw::current_allocator();
  hipStream_t stream = nullptr;
  void* x = nullptr;
  void* y = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  FILE* json = nullptr;
  ~Bufs() {
    if (x || y || ws) (void)hipStreamSynchronize(stream);
    uw::free_with(a, x);
    uw::free_with(a, y);
    uw::free_with(a, ws);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (json) std::fclose(json);
  }
};

bool feasible(const uw_matrix* m, int p) {
  return p == UW_PIPE_PALETTE_DIRECT ? m->pidx != nullptr : m->stream != nullptr;
}

// n values from N(0,1) as BF16 bit patterns: a 64-bit xorshift generator,
// Box-Muller, then round to nearest even from fp32 (x has no NaNs).
std::vector<uint16_t> normal_bf16(size_t n, uint64_t seed) {
  std::vector<uint16_t> out(n);
  uint64_t st = seed ? seed : 0x9E3779B97F4A7C15ull;
  auto next = [&]() {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
  };
  for (size_t i = 0; i < n; i += 2) {
    const double u1 = ((next() >> 11) + 1.0) * 0x1.0p-53;   // (0, 1]
    const double u2 = (next() >> 11) * 0x1.0p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    const float v[2] = {(float)(r * std::cos(6.283185307179586 * u2)), (float)(r * std::sin(6.283185307179586 * u2))};
    for (int t = 0; t < 2 && i + t < n; ++t) {
      uint32_t b;
      std::memcpy(&b, &v[t], 4);
      b += 0x7FFFu + ((b >> 16) & 1u);
      out[i + t] = (uint16_t)(b >> 16);
    }
  }
  return out;
}

}  // namespace

extern "C" uw_status uw_autotune(const uw_matrix* const* ms, const int32_t* proj, int count, int nproj,
                                 const int64_t* batches, int nb, int max_passes, const char* json_path,
                                 uw_tune_entry* out, void* stream) {
  if (!ms || !proj || count <= 0 || nproj <= 0 || !batches || nb <= 0) return UW_ERR_INVALID;
  for (int i = 0; i < count; ++i) {
    if (!ms[i] || proj[i] < 0 || proj[i] >= nproj) return UW_ERR_INVALID;
    if (ms[i]->fp8) return UW_ERR_UNSUPPORTED;
  }
  // a projection's matrices share shape, layout and residency: the choice is
  // recorded under that key
  std::vector<int> first((size_t)nproj, -1);
  for (int i = 0; i < count; ++i) {
    int& f = first[(size_t)proj[i]];
    if (f < 0) {
      f = i;
      continue;
    }
    const uw_matrix* a = ms[f];
    const uw_matrix* b = ms[i];
    if (a->rows != b->rows || a->cols != b->cols || a->layout != b->layout ||
        uw::residency_of(a) != uw::residency_of(b))
      return UW_ERR_INVALID;
  }
  for (int b = 0; b < nb; ++b)
    if (batches[b] <= 0) return UW_ERR_INVALID;
  if (max_passes <= 0) max_passes = 3;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return UW_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return UW_ERR_DEVICE;
  const int cus = prop.multiProcessorCount;

  // shared x (max K) and y (max N) for the largest batch; x ~ N(0,1) in BF16
  int64_t maxb = 0;
  uint64_t maxk = 0, maxn = 0;
  for (int b = 0; b < nb; ++b) maxb = std::max(maxb, batches[b]);
  uw_info inf;
  for (int i = 0; i < count; ++i) {
    uw_get_info(ms[i], &inf);
    maxk = std::max<uint64_t>(maxk, inf.k);
    maxn = std::max<uint64_t>(maxn, inf.n);
  }
  Bufs bufs;
  bufs.stream = s;
  uw_status ast = uw::alloc_with(bufs.a, &bufs.x, (size_t)maxb * maxk * 2 + 256);
  if (ast != UW_OK) return ast;
  ast = uw::alloc_with(bufs.a, &bufs.y, (size_t)maxb * maxn * 4 + 256);
  if (ast != UW_OK) return ast;
  {
    const std::vector<uint16_t> xh = normal_bf16((size_t)maxb * maxk, 0x5555000000000001ull);
    if (hipMemcpyAsync(bufs.x, xh.data(), xh.size() * 2, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return UW_ERR_DEVICE;
  }
  if (hipEventCreate(&bufs.e0) != hipSuccess || hipEventCreate(&bufs.e1) != hipSuccess) return UW_ERR_DEVICE;
  const hipEvent_t e0 = bufs.e0, e1 = bufs.e1;
  std::vector<uw_job> jobs((size_t)count);
  FILE* jf = nullptr;
  if (json_path) {
    jf = bufs.json = std::fopen(json_path, "w");
    if (!jf) return UW_ERR_INVALID;
    std::fprintf(jf, "{\n  \"entries\": [\n");
  }
  bool first_entry = true;
  uw_status result = UW_OK;

  for (int bi = 0; bi < nb && result == UW_OK; ++bi) {
    const int64_t batch = batches[bi];
    std::vector<Choice> cfg((size_t)nproj);
    for (int p = 0; p < nproj; ++p) {
      bool all_direct = true;
      for (int i = 0; i < count; ++i)
        if (proj[i] == p && !feasible(ms[i], UW_PIPE_PALETTE_DIRECT)) all_direct = false;
      cfg[(size_t)p].pipeline = all_direct ? UW_PIPE_PALETTE_DIRECT : UW_PIPE_EXPONENT;
    }
    // time one pass of the sequence under a configuration (microseconds)
    auto measure = [&](const std::vector<Choice>& c, double* us) -> uw_status {
      for (int i = 0; i < count; ++i) {
        uw_job& j = jobs[(size_t)i];
        const Choice& ch = c[(size_t)proj[i]];
        j.m = ms[i];
        j.pipeline = ch.pipeline;
        j.cfg.variant = ch.variant;
        j.cfg.split_k = ch.split_k;
        j.cfg.decode_cus = ch.decode_cus;
        j.cfg.reserved = 0;
        j.x_dev = static_cast<const uint16_t*>(bufs.x);
        j.y_dev = static_cast<float*>(bufs.y);
        j.batch = batch;
      }
      size_t need = 0;
      uw_status st = uw::jobs_workspace(jobs.data(), count, &need);
      if (st != UW_OK) return st;
      if (need > bufs.ws_bytes) {
        uw::free_with(bufs.a, bufs.ws);
        bufs.ws = nullptr;
        bufs.ws_bytes = 0;
        st = uw::alloc_with(bufs.a, &bufs.ws, need);
        if (st != UW_OK) return st;
        bufs.ws_bytes = need;
      }
      double t[3];
      for (int r = -1; r < 3; ++r) {
        if (hipEventRecord(e0, s) != hipSuccess) return UW_ERR_DEVICE;
        st = uw::run_jobs(jobs.data(), count, 0, bufs.ws, bufs.ws_bytes, s);
        if (st != UW_OK) return st;
        if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return UW_ERR_DEVICE;
        float ms_ = 0.f;
        if (hipEventElapsedTime(&ms_, e0, e1) != hipSuccess) return UW_ERR_DEVICE;
        if (r >= 0) t[r] = 1e3 * (double)ms_;
      }
      std::sort(t, t + 3);
      *us = t[1];
      return UW_OK;
    };

    double best = 0;
    result = measure(cfg, &best);
    if (result != UW_OK) break;
    // A candidate that measured 1 % faster is measured again right after the
    // incumbent: the chip's clock drifts as it heats, so two times taken far
    // apart compare clocks as much as kernels (the same kernel has measured
    // 10-20 % apart in back-to-back runs).  It replaces the incumbent only if
    // it is still 1 % faster; the incumbent's new time is the reference
    // either way.  Sets result on a device error.
    auto confirm = [&](const std::vector<Choice>& trial, double* t) -> bool {
      double tb = 0, t2 = 0;
      result = measure(cfg, &tb);
      if (result != UW_OK) return false;
      result = measure(trial, &t2);
      if (result != UW_OK) return false;
      if (t2 < tb * 0.99) {
        *t = t2;
        return true;
      }
      best = tb;
      return false;
    };
    const int nvar = uw_variant_count();
    for (int pass = 0; pass < max_passes && result == UW_OK; ++pass) {
      bool improved = false;
      for (int p = 0; p < nproj && result == UW_OK; ++p) {   // gate, then up, then down
        std::vector<Choice> cands;
        for (int pl = UW_PIPE_FULL; pl <= UW_PIPE_PALETTE_DIRECT; ++pl) {
          bool ok = true;
          for (int i = 0; i < count; ++i)
            if (proj[i] == p && !feasible(ms[i], pl)) ok = false;
          if (!ok) continue;
          bool all_nk = true;
          for (int i = 0; i < count; ++i)
            if (proj[i] == p && ms[i]->layout != 0) all_nk = false;
          for (int v = 1; v <= nvar; ++v) {
            if (!uw::gemm_variant_supported(v, all_nk ? 0 : 1)) continue;   // [N][K]-only kernels
            int bm = 0, bn = 0;
            const int tile = uw::gemm_variant_tile(v);
            if (tile >= 0) uw::mfma2_tile_dims(tile, &bm, &bn);
            if (v == 1 && batch > 32) continue;                 // the VALU kernel only for small batches
            if (bm > 32 && batch < 8) continue;                 // 64- to 256-row tiles from batch 8 on
            if (bm == 32 && (batch < 2 || batch > 128)) continue;   // 32-row tiles for batches 2..128
            if (bm == 512 && batch < 256) continue;                 // the 512-row tile from batch 256
            if (tile >= uw::mfma2_late_first() && bm == 256 && batch < 128) continue;   // its 256-row version from 128
            if (uw::gemm_variant_is_rf(v) && batch > 2 * uw::mfma_rf_max_batch()) continue;   // <= 128 rows
            Choice c;
            c.pipeline = pl;
            c.variant = v;
            cands.push_back(c);
          }
        }
        // stage 1: pipeline x variant, no split
        for (const Choice& c : cands) {
          if (c == cfg[(size_t)p]) continue;
          std::vector<Choice> trial = cfg;
          trial[(size_t)p] = c;
          double t = 0;
          result = measure(trial, &t);
          if (result != UW_OK) break;
          if (t < best * 0.99 && confirm(trial, &t)) {
            best = t;
            cfg = trial;
            improved = true;
          }
          if (result != UW_OK) break;
        }
        // stage 1b: the preprocessing pipelines again, with preprocessing of
        // the next matrix running beside the GEMM on every CU
        for (const Choice& c0 : cands) {
          if (result != UW_OK) break;
          if (c0.pipeline == UW_PIPE_PALETTE_DIRECT) continue;
          Choice c = c0;
          c.decode_cus = cus;
          if (c == cfg[(size_t)p]) continue;
          std::vector<Choice> trial = cfg;
          trial[(size_t)p] = c;
          double t = 0;
          result = measure(trial, &t);
          if (result != UW_OK) break;
          if (t < best * 0.99 && confirm(trial, &t)) {
            best = t;
            cfg = trial;
            improved = true;
          }
          if (result != UW_OK) break;
        }
        // stage 1c: the K split of the chosen kernel (0 = the library's rule;
        // 1 = no split); the register-fed, LDS-tiled and [K][N] GEMV kernels
        // take it, the [N][K] GEMV ignores it
        if (result == UW_OK) {
          const Choice base = cfg[(size_t)p];
          bool splits = true;
          if (base.variant == 1 || (base.variant <= 0 && batch <= 4)) {
            for (int i = 0; i < count; ++i)
              if (proj[i] == p && ms[i]->layout == 0) splits = false;
          }
          for (int sk : {1, 2, 4, 8}) {
            if (!splits) break;
            Choice c = base;
            c.split_k = sk;
            if (c == cfg[(size_t)p]) continue;
            std::vector<Choice> trial = cfg;
            trial[(size_t)p] = c;
            double t = 0;
            result = measure(trial, &t);
            if (result != UW_OK) break;
            if (t < best * 0.99 && confirm(trial, &t)) {
              best = t;
              cfg = trial;
              improved = true;
            }
            if (result != UW_OK) break;
          }
        }
        // stage 2: CUs for the preprocessing kernel of the chosen pipeline
        if (result == UW_OK && cfg[(size_t)p].pipeline != UW_PIPE_PALETTE_DIRECT) {
          for (int frac : {8, 4, 2}) {
            Choice c = cfg[(size_t)p];
            c.decode_cus = (cus / frac) / 8 * 8;   // whole CUs per XCD stripe
            if (c.decode_cus <= 0 || c == cfg[(size_t)p]) continue;
            std::vector<Choice> trial = cfg;
            trial[(size_t)p] = c;
            double t = 0;
            result = measure(trial, &t);
            if (result != UW_OK) break;
            if (t < best * 0.99 && confirm(trial, &t)) {
              best = t;
              cfg = trial;
              improved = true;
            }
            if (result != UW_OK) break;
          }
        }
      }
      if (!improved) break;
    }
    if (result != UW_OK) break;
    for (int p = 0; p < nproj; ++p) {
      const Choice& c = cfg[(size_t)p];
      const int fi = first[(size_t)p];
      uw_tune_entry e;
      std::memset(&e, 0, sizeof(e));
      e.batch = batch;
      e.projection = p;
      e.pipeline = c.pipeline;
      e.variant = c.variant;
      e.split_k = c.split_k;
      e.decode_cus = c.decode_cus;
      if (fi >= 0) {
        uw_get_info(ms[fi], &inf);
        e.layout = (int32_t)inf.layout;
        e.n = inf.n;
        e.k = inf.k;
        e.residency = uw::residency_of(ms[fi]);
      }
      e.sequence_us = best;
      if (out) out[(size_t)bi * (size_t)nproj + (size_t)p] = e;
      if (jf && fi >= 0) {
        std::fprintf(jf, "%s    {\"batch\": %lld, \"projection\": %d, \"n\": %llu, \"k\": %llu, \"layout\": %d, "
                         "\"residency\": %d, \"pipeline\": %d, \"variant\": %d, \"split_k\": %d, "
                         "\"decode_cus\": %d, \"sequence_us\": %.2f}",
                     first_entry ? "" : ",\n", (long long)batch, p, (unsigned long long)e.n,
                     (unsigned long long)e.k, e.layout, e.residency, c.pipeline, c.variant, c.split_k,
                     c.decode_cus, best);
        first_entry = false;
      }
    }
  }
  if (jf) {
    std::fprintf(jf, "\n  ]\n}\n");
    bufs.json = nullptr;
    if (std::fclose(jf) != 0 && result == UW_OK) result = UW_ERR_INVALID;
  }
  return result;
}

// Grouped calls (gate+up, q+k+v): one choice for the whole call, measured on
// uw_matmul_reconstruct_grouped itself, since a group runs kernels of its own
// (the grouped GEMV and the grouped LDS tile, which split K over the group's
// tiles together) whose best configuration is not either matrix's.  No
// coordinate descent: the call has one choice, so every candidate is timed.
extern "C" uw_status uw_autotune_grouped(const uw_matrix* const* ms, int group, int ngroups,
                                         const int64_t* batches, int nb, const char* json_path,
                                         uw_tune_entry* out, void* stream) {
  if (!ms || group < 2 || group > uw::kTuneGroupMax || ngroups <= 0 || !batches || nb <= 0) return UW_ERR_INVALID;
  const int count = group * ngroups;
  for (int i = 0; i < count; ++i) {
    if (!ms[i]) return UW_ERR_INVALID;
    if (ms[i]->fp8) return UW_ERR_UNSUPPORTED;
  }
  // one table key per group: its matrices share K, layout and residency, and
  // every group matches the first matrix for matrix
  for (int i = 0; i < count; ++i) {
    const uw_matrix* a = ms[i % group];
    const uw_matrix* b = ms[i];
    const uw_matrix* g0 = ms[0];
    if (a->rows != b->rows || a->cols != b->cols || a->layout != b->layout ||
        uw::residency_of(a) != uw::residency_of(b) || b->layout != g0->layout ||
        uw::residency_of(b) != uw::residency_of(g0))
      return UW_ERR_INVALID;
  }
  uw_info inf;
  uint64_t k = 0, ntot = 0;
  for (int i = 0; i < group; ++i) {
    uw_get_info(ms[i], &inf);
    if (i == 0) k = inf.k;
    if (inf.k != k) return UW_ERR_INVALID;
    ntot += inf.n;
  }
  const int layout = (int)ms[0]->layout;
  const int residency = uw::residency_of(ms[0]);
  int64_t maxb = 0;
  for (int b = 0; b < nb; ++b) {
    if (batches[b] <= 0) return UW_ERR_INVALID;
    maxb = std::max(maxb, batches[b]);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);

  Bufs bufs;
  bufs.stream = s;
  uw_status st = uw::alloc_with(bufs.a, &bufs.x, (size_t)maxb * k * 2 + 256);
  if (st != UW_OK) return st;
  st = uw::alloc_with(bufs.a, &bufs.y, (size_t)maxb * ntot * 4 + 256);
  if (st != UW_OK) return st;
  {
    const std::vector<uint16_t> xh = normal_bf16((size_t)maxb * k, 0x5555000000000003ull);
    if (hipMemcpyAsync(bufs.x, xh.data(), xh.size() * 2, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return UW_ERR_DEVICE;
  }
  if (hipEventCreate(&bufs.e0) != hipSuccess || hipEventCreate(&bufs.e1) != hipSuccess) return UW_ERR_DEVICE;
  FILE* jf = nullptr;
  if (json_path) {
    jf = bufs.json = std::fopen(json_path, "w");
    if (!jf) return UW_ERR_INVALID;
    std::fprintf(jf, "{\n  \"entries\": [\n");
  }

  // one pass of grouped calls over the groups under a choice (microseconds);
  // UW_ERR_UNSUPPORTED when the choice cannot run
  auto measure = [&](const Choice& c, int64_t batch, double* us) -> uw_status {
    uw_kernel_cfg cfg;
    cfg.variant = c.variant;
    cfg.split_k = c.split_k;
    cfg.decode_cus = c.decode_cus;
    cfg.reserved = 0;
    size_t need = 0;
    uw_status r = uw_workspace_size_grouped(ms, group, (uw_pipeline)c.pipeline, batch, &cfg, &need);
    if (r != UW_OK) return r;
    if (need > bufs.ws_bytes) {
      uw::free_with(bufs.a, bufs.ws);
      bufs.ws = nullptr;
      bufs.ws_bytes = 0;
      r = uw::alloc_with(bufs.a, &bufs.ws, need);
      if (r != UW_OK) return r;
      bufs.ws_bytes = need;
    }
    double t[3];
    for (int rep = -1; rep < 3; ++rep) {
      if (hipEventRecord(bufs.e0, s) != hipSuccess) return UW_ERR_DEVICE;
      for (int g = 0; g < ngroups; ++g) {
        r = uw_matmul_reconstruct_grouped(ms + (size_t)g * group, group, (uw_pipeline)c.pipeline,
                                          static_cast<const uint16_t*>(bufs.x), batch, static_cast<float*>(bufs.y),
                                          bufs.ws, bufs.ws_bytes, &cfg, stream);
        if (r != UW_OK) return r;
      }
      if (hipEventRecord(bufs.e1, s) != hipSuccess || hipEventSynchronize(bufs.e1) != hipSuccess)
        return UW_ERR_DEVICE;
      float ms_ = 0.f;
      if (hipEventElapsedTime(&ms_, bufs.e0, bufs.e1) != hipSuccess) return UW_ERR_DEVICE;
      if (rep >= 0) t[rep] = 1e3 * (double)ms_;
    }
    std::sort(t, t + 3);
    *us = t[1];
    return UW_OK;
  };

  const int nvar = uw_variant_count();
  bool first_entry = true;
  for (int bi = 0; bi < nb; ++bi) {
    const int64_t batch = batches[bi];
    std::vector<Choice> cands;
    for (int pl = UW_PIPE_FULL; pl <= UW_PIPE_PALETTE_DIRECT; ++pl) {
      bool ok = true;
      for (int i = 0; i < group; ++i) ok = ok && feasible(ms[i], pl);
      if (!ok) continue;
      for (int v = 0; v <= nvar; ++v) {
        if (v > 0 && !uw::gemm_variant_supported(v, layout)) continue;
        int bm = 0, bn = 0;
        const int tile = uw::gemm_variant_tile(v);
        if (tile >= 0) uw::mfma2_tile_dims(tile, &bm, &bn);
        if (v == 1 && batch > 32) continue;                     // the same filters as uw_autotune
        if (bm > 32 && batch < 8) continue;
        if (bm == 32 && (batch < 2 || batch > 128)) continue;
        if (bm == 512 && batch < 256) continue;
        if (tile >= uw::mfma2_late_first() && bm == 256 && batch < 128) continue;
        if (uw::gemm_variant_is_rf(v) && batch > 2 * uw::mfma_rf_max_batch()) continue;
        Choice c;
        c.pipeline = pl;
        c.variant = v;
        cands.push_back(c);
      }
    }
    Choice best_c;
    double best = -1;
    // a faster-looking candidate is timed again right after the incumbent
    // (the clock drifts as the chip heats; see uw_autotune)
    auto confirm = [&](const Choice& c, double* t) -> uw_status {
      double tb = 0, t2 = 0;
      uw_status r = measure(best_c, batch, &tb);
      if (r != UW_OK) return r;
      r = measure(c, batch, &t2);
      if (r != UW_OK) return r;
      if (t2 < tb * 0.99) {
        *t = t2;
      } else {
        best = tb;
        *t = -1;
      }
      return UW_OK;
    };
    for (const Choice& c : cands) {
      double t = 0;
      st = measure(c, batch, &t);
      if (st == UW_ERR_UNSUPPORTED) continue;
      if (st != UW_OK) return st;
      if (best >= 0 && t < best * 0.99) {
        st = confirm(c, &t);
        if (st != UW_OK) return st;
      }
      if (best < 0 || (t >= 0 && t < best * 0.99)) {
        best = t;
        best_c = c;
      }
    }
    if (best < 0) return UW_ERR_UNSUPPORTED;
    // the K split of the fastest (0 = the library's rule, 1 = none)
    const Choice base = best_c;
    for (int sk : {1, 2, 4, 8}) {
      Choice c = base;
      c.split_k = sk;
      double t = 0;
      st = measure(c, batch, &t);
      if (st == UW_ERR_UNSUPPORTED) continue;
      if (st != UW_OK) return st;
      if (t < best * 0.99) {
        st = confirm(c, &t);
        if (st != UW_OK) return st;
      }
      if (t >= 0 && t < best * 0.99) {
        best = t;
        best_c = c;
      }
    }
    uw_tune_entry e;
    std::memset(&e, 0, sizeof(e));
    e.batch = batch;
    e.projection = 0;
    e.pipeline = best_c.pipeline;
    e.variant = best_c.variant;
    e.split_k = best_c.split_k;
    e.decode_cus = 0;
    e.layout = layout;
    e.residency = residency;
    e.group = group;
    e.n = ntot;
    e.k = k;
    e.sequence_us = best;
    if (out) out[bi] = e;
    if (jf) {
      std::fprintf(jf, "%s    {\"batch\": %lld, \"projection\": 0, \"group\": %d, \"n\": %llu, \"k\": %llu, "
                       "\"layout\": %d, \"residency\": %d, \"pipeline\": %d, \"variant\": %d, \"split_k\": %d, "
                       "\"decode_cus\": 0, \"sequence_us\": %.2f}",
                   first_entry ? "" : ",\n", (long long)batch, group, (unsigned long long)ntot,
                   (unsigned long long)k, layout, residency, e.pipeline, e.variant, e.split_k, best);
      first_entry = false;
    }
  }
  if (jf) {
    std::fprintf(jf, "\n  ]\n}\n");
    bufs.json = nullptr;
    if (std::fclose(jf) != 0) return UW_ERR_INVALID;
  }
  return UW_OK;
}
