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
// three runs after a warm-up.  Candidates per projection: every pipeline all
// its matrices can run (direct palette needs resident indices, the others the
// Huffman stream) x every GEMM variant that suits the batch; then, for a
// pipeline with preprocessing, the CUs given to the preprocessing kernel.
#include <algorithm>
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

struct Bufs {
  void* x = nullptr;
  void* y = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  ~Bufs() {
    if (x) (void)hipFree(x);
    if (y) (void)hipFree(y);
    if (ws) (void)hipFree(ws);
  }
};

bool feasible(const uw_matrix* m, int p) {
  return p == UW_PIPE_PALETTE_DIRECT ? m->pidx != nullptr : m->stream != nullptr;
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
  for (int b = 0; b < nb; ++b)
    if (batches[b] <= 0) return UW_ERR_INVALID;
  if (max_passes <= 0) max_passes = 3;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return UW_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return UW_ERR_DEVICE;
  const int cus = prop.multiProcessorCount;

  // shared x (max K) and y (max N) for the largest batch; contents are zero
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
  if (hipMalloc(&bufs.x, (size_t)maxb * maxk * 2 + 256) != hipSuccess) return UW_ERR_NOMEM;
  if (hipMalloc(&bufs.y, (size_t)maxb * maxn * 4 + 256) != hipSuccess) return UW_ERR_NOMEM;
  if (hipMemsetAsync(bufs.x, 0, (size_t)maxb * maxk * 2, s) != hipSuccess) return UW_ERR_DEVICE;

  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return UW_ERR_DEVICE;
  std::vector<uw_job> jobs((size_t)count);
  FILE* jf = json_path ? std::fopen(json_path, "w") : nullptr;
  if (json_path && !jf) return UW_ERR_INVALID;
  if (jf) std::fprintf(jf, "{\n  \"entries\": [\n");
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
      uw_status st = uw_sequence_workspace_size(jobs.data(), count, &need);
      if (st != UW_OK) return st;
      if (need > bufs.ws_bytes) {
        if (bufs.ws) (void)hipFree(bufs.ws);
        bufs.ws = nullptr;
        bufs.ws_bytes = 0;
        if (hipMalloc(&bufs.ws, need) != hipSuccess) return UW_ERR_NOMEM;
        bufs.ws_bytes = need;
      }
      double t[3];
      for (int r = -1; r < 3; ++r) {
        if (hipEventRecord(e0, s) != hipSuccess) return UW_ERR_DEVICE;
        st = uw_run_sequence(jobs.data(), count, 0, bufs.ws, bufs.ws_bytes, s);
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
          const int rf = uw::rf_first_variant();                  // the register-fed MFMA kernels
          bool all_nk = true;
          for (int i = 0; i < count; ++i)
            if (proj[i] == p && ms[i]->layout != 0) all_nk = false;
          for (int v = 1; v <= nvar; ++v) {
            int bm = 0, bn = 0;
            if (v > 1 && v < rf) uw::mfma2_tile_dims(v - 2, &bm, &bn);
            if (v == 1 && batch > 32) continue;                 // the VALU kernel only for small batches
            if (bm > 32 && batch < 8) continue;                 // 64- to 256-row tiles from batch 8 on
            if (bm == 32 && (batch < 2 || batch > 128)) continue;   // 32-row tiles for batches 2..128
            if (v >= rf && (!all_nk || batch > 2 * uw::mfma_rf_max_batch())) continue;   // [N][K] only, <= 128 rows
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
          if (t < best * 0.99) {
            best = t;
            cfg = trial;
            improved = true;
          }
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
          if (t < best * 0.99) {
            best = t;
            cfg = trial;
            improved = true;
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
            if (t < best * 0.99) {
              best = t;
              cfg = trial;
              improved = true;
            }
          }
        }
      }
      if (!improved) break;
    }
    if (result != UW_OK) break;
    for (int p = 0; p < nproj; ++p) {
      const Choice& c = cfg[(size_t)p];
      if (out) {
        uw_tune_entry& e = out[(size_t)bi * (size_t)nproj + (size_t)p];
        e.batch = batch;
        e.projection = p;
        e.pipeline = c.pipeline;
        e.variant = c.variant;
        e.split_k = c.split_k;
        e.decode_cus = c.decode_cus;
        e.sequence_us = best;
      }
      if (jf) {
        std::fprintf(jf, "%s    {\"batch\": %lld, \"projection\": %d, \"pipeline\": %d, \"variant\": %d, "
                         "\"split_k\": %d, \"decode_cus\": %d, \"sequence_us\": %.2f}",
                     first_entry ? "" : ",\n", (long long)batch, p, c.pipeline, c.variant, c.split_k,
                     c.decode_cus, best);
        first_entry = false;
      }
    }
  }
  if (jf) {
    std::fprintf(jf, "\n  ]\n}\n");
    std::fclose(jf);
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return result;
}
