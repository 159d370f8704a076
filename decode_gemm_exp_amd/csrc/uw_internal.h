// uw_internal.h -- shared declarations of libunweight's host code and kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/unweight.h"

namespace uw {

constexpr int kGroup = 64;        // weights per verbatim decision
constexpr int kPal = 16;          // palette entries
constexpr int kMaxLen = 12;       // longest codeword
constexpr int kLutBits = 12;      // decode table index width (4096 entries)
// Decode table entry for a 12-bit window, two words:
//   word 0: bits 0-4 the bits its whole codewords take (bit 5 clear, so a
//           64-bit shift can take the word as its count), bits 8-15 four
//           times the codeword count (up to 8), bit 16 set when no codeword
//           starts in the window (a one-symbol code only);
//   word 1: the codewords' slots as nibbles, first codeword lowest.
constexpr int kLutWords = 2;
constexpr uint32_t kLutBytes = 4u * kLutWords << kLutBits;   // 32 KB
constexpr uint32_t kLutInvalid = 1u << 16;
constexpr uint64_t kHeaderBytes = 2304;

// Host-side tables of one matrix (all tiny).
struct Tables {
  uint64_t hist[256];
  uint32_t palette_size;
  uint8_t palette[kPal];
  int16_t slot_of[256];           // -1 = not in palette
  uint64_t coded_count[kPal];
  uint32_t n_coded;
  uint8_t code_len[kPal];
  uint16_t code[kPal];
};

}  // namespace uw

struct uw_matrix {
  int device = 0;
  uint32_t layout = 0, seg_groups = 4;
  uint64_t rows = 0, cols = 0, numel = 0, groups = 0, segments = 0, flag_words = 0;
  uint64_t V = 0, W = 0, code_bits = 0;
  uw::Tables t{};
  // device sections
  uint8_t* sm = nullptr;          // numel (BF16) or numel / 2 (FP8) bytes
  uint32_t* vflags = nullptr;     // flag_words
  uint32_t* vrank = nullptr;      // flag_words
  uint8_t* vexp = nullptr;        // 64 * V (may be null when V == 0)
  uint32_t* seg_off = nullptr;    // segments + 1
  uint32_t* stream = nullptr;     // W + 2
  uint32_t* lut = nullptr;        // 4096 decode entries of kLutWords words
  uint8_t* pidx = nullptr;        // resident palette indices (numel / 2) or null
  int* corrupt = nullptr;         // device flag set by decoders
  uint32_t wave_span = 0;         // most stream words any 64-segment wave covers (from a 4-word boundary)
  bool fp8 = false;               // FP8 E4M3 weights: sm holds numel / 2 bytes of sign+mantissa nibbles
  uw_allocator alloc{};           // the hooks its sections came from (alloc == NULL: hipMalloc)
};

namespace uw {

// ---- tables.cpp --------------------------------------------------------------
void choose_palette(Tables& t);                        // from t.hist
bool limited_lengths(const uint64_t* w, int n, int lmax, uint8_t* len);
void assign_codes(Tables& t);                          // from code_len
void build_decode_lut(const Tables& t, uint32_t* lut);   // kLutWords << kLutBits words

// Compute units of the current device (256 if the query fails).
int device_cus();

// ---- runtime.cpp: allocator, sequence-runner HIP objects, tuned choices -------
uw_allocator current_allocator();
// bytes of device memory from allocator a (hipMalloc when a.alloc is NULL);
// UW_ERR_NOMEM when a hook returns NULL, UW_ERR_INVALID when its block is not
// 256-byte aligned
uw_status alloc_with(const uw_allocator& a, void** p, size_t bytes);
void free_with(const uw_allocator& a, void* p);
struct SplitStreams {
  hipStream_t dec = nullptr, gemm = nullptr;
};
// the stream pair of the current device for a decode share of `decode_cus`
// CUs (>= the CU count: two unmasked streams); owned by the library
uw_status split_streams(int decode_cus, SplitStreams* out);
// held by uw_run_sequence for its whole call
std::mutex& sequence_mutex();
// at least `count` events of the current device; caller holds sequence_mutex()
uw_status pooled_events(size_t count, hipEvent_t** out);
// the sequence runner on jobs as given (api.cpp): explicit pipelines, cfgs
// used as they are; uw_run_sequence resolves UW_PIPE_AUTO and tuned cfgs first
uw_status jobs_workspace(const uw_job* jobs, int count, size_t* bytes);
uw_status run_jobs(const uw_job* jobs, int count, int32_t decode_cus, void* ws, size_t ws_bytes, hipStream_t s);
// the GEMM stage of uw_matmul_stage with its partial sums in `part`
// (part_bytes); *need = the bytes the call needs, set before the size check
uw_status matmul_stage_into(const uw_matrix* m, int p, const void* prep, const uint16_t* x, int64_t batch, float* y,
                            void* part, size_t part_bytes, const uw_kernel_cfg* cfg, hipStream_t s, size_t* need);
// bit 0: Huffman stream resident, bit 1: palette indices resident
int residency_of(const uw_matrix* m);
// the tuned choice for a shape, residency, group (0: one matrix; g >= 2: a
// grouped call on g matrices of total N n) and batch (nearest tuned batch on
// a log scale); false when the table holds none
bool tuned_lookup(uint64_t n, uint64_t k, int layout, int residency, int64_t batch, uw_tune_entry* out,
                  int group = 0);
constexpr int kTuneGroupMax = 64;

// uw_set_kernel_events: record the caller's events around a main kernel's
// launch on stream s (nothing when none are set)
void kernel_event_before(hipStream_t s);
void kernel_event_after(hipStream_t s);

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once
// per (kernel, device, size); thread safe (api.cpp).
hipError_t allow_dynamic_lds(const void* kernel, int bytes);

// ---- kernel launchers (compress.hip, decode.hip, gemm*.hip) ------------------
hipError_t launch_fp8_fields(const uint8_t* w, uint64_t numel, uint16_t* out, hipStream_t s);
hipError_t launch_fp8_pack(const uint8_t* w, uint64_t numel, uint8_t* out, hipStream_t s);
hipError_t launch_histogram(const uint16_t* w, uint64_t numel, uint32_t* hist, hipStream_t s);
hipError_t launch_flags(const uint16_t* w, uint64_t numel, uint64_t groups, const uint8_t* slot_tab,
                        uint8_t* sm, uint32_t* vflags, uint32_t* coded, hipStream_t s);
hipError_t launch_rank_scan(const uint32_t* vflags, uint64_t words, uint32_t* vrank,
                            uint64_t* total, uint64_t* tiles_ws, hipStream_t s);
uint64_t scan_tiles(uint64_t n);   // u64 tile sums a scan of n values needs
hipError_t launch_segment_bits(const uint16_t* w, uint64_t groups, uint32_t seg_groups,
                               uint64_t segments, const uint8_t* len_tab, const uint32_t* vflags,
                               uint32_t* seg_words, hipStream_t s);
hipError_t launch_offsets_scan(const uint32_t* seg_words, uint64_t segments, uint32_t* seg_off,
                               uint64_t* tiles_ws, hipStream_t s);
hipError_t launch_wave_span(const uint32_t* seg_off, uint64_t segments, uint32_t* out, hipStream_t s);
hipError_t launch_encode(const uint16_t* w, uint64_t groups, uint32_t seg_groups, uint64_t segments,
                         const uint32_t* codebook, const uint32_t* vflags, const uint32_t* vrank,
                         const uint32_t* seg_off, uint32_t* stream, uint8_t* vexp, hipStream_t s);

// The palette as seen by kernels: 16 exponent bytes in 4 words; when its
// entries are consecutive exponents, run = 1 and base4 = first entry x 0x01010101.
struct PalView {
  uint32_t w[4];
  uint32_t run;
  uint32_t base4;
};

enum DecodeMode { kDecodeNibble = 0, kDecodeExponent = 1, kDecodeFull = 2, kDecodeFp8 = 3 };
struct DecodeArgs {
  const uint32_t* stream; uint64_t stream_words;   // including slack
  const uint32_t* seg_off;
  const uint32_t* vflags; const uint32_t* vrank; const uint8_t* vexp;
  uint64_t vexp_bytes;                              // 64 x verbatim groups
  const uint8_t* sm;
  const uint32_t* lut;
  PalView pal;
  uint64_t len_pack;                                // 4-bit code length per slot
  uint64_t groups, segments; uint32_t seg_groups;
  uint32_t wave_span;                               // see uw_matrix::wave_span
  void* out;
  int* corrupt;
};
hipError_t launch_decode(const DecodeArgs& a, int mode, hipStream_t s);

// weight formats seen by the GEMM kernels
// kFmtPalRun: palette formats whose entries are consecutive exponents (the
// lookup is a bytewise add); a separate format keeps kernels branch-free
enum WFmt { kFmtBf16 = 0, kFmtExp = 1, kFmtPal = 2, kFmtPalRun = 3 };
constexpr bool fmt_is_pal(int f) { return f == kFmtPal || f == kFmtPalRun; }
struct WeightView {
  int fmt;
  int layout;                       // 0 = stored [N][K], 1 = stored [K][N]
  uint64_t n, k;                    // logical
  const uint16_t* bf16;             // kFmtBf16
  const uint8_t* sm;                // kFmtExp / kFmtPal
  const uint8_t* ex;                // kFmtExp: exponent bytes
  const uint8_t* pidx;              // kFmtPal
  const uint32_t* vflags; const uint32_t* vrank; const uint8_t* vexp;   // kFmtPal
  uint64_t vexp_bytes;              // kFmtPal: 64 x verbatim groups
  PalView pal;
};
// y[:, col0 : col0+n] of a row-major [batch][ldy] output
hipError_t launch_gemm(const WeightView& w, const uint16_t* x, int64_t batch, float* y,
                       int64_t ldy, int64_t col0, const uw_kernel_cfg* cfg, float* partial,
                       size_t partial_elems, hipStream_t s);
size_t gemm_partial_elems(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg);
// one launch for up to 4 stored [N][K] matrices sharing K and x that resolve
// to the VALU GEMV; hipErrorNotSupported otherwise
hipError_t launch_gemm_group(const WeightView* ws, int count, const uint16_t* x, int64_t batch, float* y,
                             int64_t ldy, const int64_t* col0s, const uw_kernel_cfg* cfg, hipStream_t s);
size_t gemm_partial_elems_max(const WeightView& w, int64_t batch, int split_k);
void describe_gemm(const WeightView& w, int64_t batch, const uw_kernel_cfg* cfg, uw_gemm_plan* out);
int gemm_variant_count();
int rf_first_variant();                          // first register-fed MFMA variant
bool gemm_variant_supported(int v, int layout);  // register-fed variants: stored [N][K] only
// y[b][col0 + n] = sum over slices p of part[p][b][n], fixed order
hipError_t launch_sum_slices(const float* part, int slices, uint64_t n, int64_t batch, float* y, int64_t ldy,
                             int64_t col0, hipStream_t s);
// gemm_mfma.hip
int mfma2_tile_count();
void mfma2_tile_dims(int tile, int* bm, int* bn);
void mfma2_tile_shape(int tile, int* waves, int* wgm, bool* xreg, int* kw);   // kw: K step in units of 64
int mfma2_late_first();   // first tile numbered after the register-fed kernels (128-wide K steps, eight-wave 128x256 and 64x128)
bool mfma2_wide_pays(const WeightView& w, int64_t batch, int tile);
bool gemm_variant_is_rf(int v);                         // a register-fed MFMA variant
int gemm_variant_tile(int v);                           // the MFMA tile of variant v, or -1
// A group of matrices in one LDS-tiled launch (same K, layout, format class)
constexpr int kMfma2GroupMax = 4;
// ... or in one grouped GEMV launch (gemm.hip)
constexpr int kGemvGroupMax = 4;
// grouped calls plan both launches over one array of weight views
static_assert(kGemvGroupMax == kMfma2GroupMax, "grouped launches share their matrix limit");
constexpr int kGroupMax = kMfma2GroupMax;
struct Mfma2Group {
  WeightView w[kMfma2GroupMax];
  int64_t ycol[kMfma2GroupMax];   // first output column of each matrix in y
  int64_t pcol[kMfma2GroupMax];   // ... in the group's partial rows (split K)
  int ntiles[kMfma2GroupMax];     // N tiles of each matrix
  int bstart[kMfma2GroupMax];     // first block (grid x) of each matrix, set at launch
  int count;
};
hipError_t launch_mfma2_group(const WeightView* ws, int count, const uint16_t* x, int64_t batch, float* y,
                              int64_t ldy, const int64_t* col0s, int tile, int split_hint, float* part,
                              size_t part_elems, hipStream_t s);
size_t mfma2_group_partial_elems(const WeightView* ws, int count, int64_t batch, int tile, int split_hint);
// Grouped matmul in one LDS-tiled launch when the group's default (or forced)
// kernel is an LDS tile: SIZE_MAX when not, else the partial floats it needs.
size_t gemm_tile_group_partial_elems(const WeightView* ws, int count, int64_t batch, const uw_kernel_cfg* cfg);
hipError_t launch_gemm_tile_group(const WeightView* ws, int count, const uint16_t* x, int64_t batch, float* y,
                                  int64_t ldy, const int64_t* col0s, const uw_kernel_cfg* cfg, float* part,
                                  size_t part_elems, hipStream_t s);
int mfma2_slices(const WeightView& w, int64_t batch, int tile, int split_hint);
size_t mfma2_partial_elems(const WeightView& w, int64_t batch, int tile, int split_hint);
hipError_t launch_mfma2(const WeightView& w, const uint16_t* x, int64_t batch, float* y, int64_t ldy, int64_t col0,
                        int tile, int split_hint, float* part, size_t part_elems, hipStream_t s);
// gemm_rf.hip (kind 0: two 16-row tiles per wave, kind 1: four; kinds 2 and
// 3: x shared through LDS, one and two tiles per wave)
int mfma_rf_kinds();
int mfma_rf_max_batch();
bool mfma_rf_supported(const WeightView& w, int kind);   // stored [N][K], flag words fit in LDS
int mfma_rf_slices(const WeightView& w, int kind, int split_hint, int cus);
size_t mfma_rf_partial_elems(const WeightView& w, int64_t batch, int kind, int split_hint, int cus);
hipError_t launch_mfma_rf(const WeightView& w, const uint16_t* x, int64_t batch, float* y, int64_t ldy,
                          int64_t col0, int kind, int split_hint, int cus, float* part, size_t part_elems,
                          hipStream_t s);

}  // namespace uw
