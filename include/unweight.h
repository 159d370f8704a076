/*
 * unweight.h -- C ABI of the MI355X (gfx950) lossless BF16 MLP-weight codec
 * and reconstructive GEMM library (libunweight.so).
 *
 * Sources, cited by page title and section heading:
 *   [EVC] "Cloudflare推出Unweight無損壓縮系統，將LLM模型大小壓縮15-22%"
 *         (easyvibecoding.app/curated/736)
 *   [GT]  goodtech.info article on Cloudflare Unweight, section
 *         "La magie du code de Huffman"
 *
 * What the library computes.  A BF16 weight matrix is split into a
 * sign+mantissa byte and an exponent byte per weight.  Exponents are coded
 * with a canonical, length-limited Huffman code over a 16-entry exponent
 * palette, and any 64-weight group holding an exponent outside the palette is
 * kept verbatim ([EVC] "BF16權重壓縮原理"; [GT]).  At inference the matrix is
 * consumed by one of four pipelines ([EVC] "四種執行管道"):
 *   UW_PIPE_FULL               Huffman decode to BF16 in HBM, then a dense GEMM
 *   UW_PIPE_EXPONENT           decode exponent bytes only, then a GEMM that
 *                              rebuilds BF16 on chip
 *   UW_PIPE_PALETTE_TRANSCODE  transcode to 4-bit palette indices at run time,
 *                              then the rebuilding GEMM
 *   UW_PIPE_PALETTE_DIRECT     indices prepared once at load (resident), the
 *                              rebuilding GEMM alone per call
 * The rebuilding GEMM fuses decompression into the matrix multiply so rebuilt
 * weights never return to HBM ([EVC] "重建矩陣乘法核心運作").
 *
 * Encoding (UWF1).  The exact stream format is fixed by this library and by
 * the independent CPU oracle that checks it; the pages leave these details
 * open.  Stored order = row-major order of the stored array; a group is 64
 * consecutive stored elements (the stored row length must be a multiple of
 * 64); the palette holds the 16 most frequent exponents (ties to the smaller
 * value) in ascending order; code lengths come from package-merge with a
 * 12-bit limit; codes are canonical and written MSB-first into little-endian
 * 32-bit words; every `seg_groups` groups form a segment that starts on a
 * word boundary; verbatim groups are absent from the stream and their 64
 * exponent bytes are kept in a side section.
 *
 * Conventions for every call.
 *   - Pointers suffixed _dev are device pointers on the current HIP device;
 *     the caller owns them.  The library never keeps them past the call.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously on it unless a call says it synchronises.
 *   - Argument and shape errors are returned before anything is enqueued.
 *   - No C++ exception crosses this interface.
 *   - A uw_matrix owns its device sections.  It may be used concurrently from
 *     several streams by calls that only read it; uw_transcode_palette with a
 *     NULL output and uw_drop_stream modify it and must not overlap any other
 *     call on the same handle.  uw_free must not be called while work on the
 *     handle is in flight.
 */
#ifndef UNWEIGHT_H_
#define UNWEIGHT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct uw_matrix uw_matrix;

typedef enum {
  UW_OK = 0,
  UW_ERR_INVALID = -1,      /* NULL pointer, negative or zero size, bad enum   */
  UW_ERR_UNSUPPORTED = -2,  /* stored row length not a multiple of 64, etc.   */
  UW_ERR_NOMEM = -3,        /* device or host allocation failed                */
  UW_ERR_DEVICE = -4,       /* a HIP runtime call failed                       */
  UW_ERR_CORRUPT = -5,      /* malformed UWF1 blob, or the decoder found an
                               invalid code / segment length (uw_sync_status) */
  UW_ERR_STATE = -6,        /* handle lacks what the call needs (e.g. the
                               Huffman stream after uw_drop_stream)            */
  UW_ERR_WORKSPACE = -7     /* workspace missing or smaller than required      */
} uw_status;

typedef enum {
  UW_LAYOUT_NK = 0,  /* stored array is W[N][K]   (K contiguous)             */
  UW_LAYOUT_KN = 1   /* stored array is W^T[K][N] (N contiguous; "transposed") */
} uw_layout;

typedef enum {
  UW_PIPE_FULL = 0,
  UW_PIPE_EXPONENT = 1,
  UW_PIPE_PALETTE_TRANSCODE = 2,
  UW_PIPE_PALETTE_DIRECT = 3,
  /* The tuned pipeline for this matrix's shape, residency and batch (see
   * uw_set_tuning / uw_load_tuning) when the table holds one that the handle
   * can run; otherwise direct palette when the indices are resident, else the
   * exponent pipeline.  ([EVC] "自動調優機制": the configuration chosen by
   * measurement is looked up per projection and batch at run time.) */
  UW_PIPE_AUTO = 15
} uw_pipeline;

typedef struct {
  uint32_t seg_groups;  /* groups per segment: power of two in [1, 64]; 0 = 4 */
  uint32_t flags;       /* reserved, must be 0                               */
} uw_compress_opts;

/* Kernel choice for one GEMM call.  Any field <= 0 means "library default".
 * Calls that take a cfg treat cfg == NULL as "the tuned choice": the kernel
 * fields of the tuning-table entry for this shape, residency and batch when
 * that entry names the pipeline the call runs, else the library default. */
typedef struct {
  int32_t variant;      /* GEMM variant (see uw_variant_count)                */
  int32_t split_k;      /* K slices of the split-K kernels                    */
  int32_t decode_cus;   /* CUs given to the preprocessing kernel when it runs
                           beside GEMMs (uw_run_sequence); 0 = no split, in
                           order on one stream; >= the device's CU count =
                           both kernels on every CU, on two unmasked streams */
  int32_t reserved;
} uw_kernel_cfg;

typedef struct {
  uint32_t layout, seg_groups;
  uint64_t rows, cols;          /* stored array shape                      */
  uint64_t n, k;                /* logical W[N][K]                         */
  uint64_t numel, groups, segments;
  uint32_t palette_size, n_coded;
  uint8_t palette[16];          /* ascending exponent values               */
  uint8_t code_len[16];         /* per palette slot, 0 = unused            */
  uint16_t code[16];            /* canonical codeword per slot             */
  uint64_t hist[256];           /* exponent histogram of all weights       */
  uint64_t coded_count[16];     /* slot counts over non-verbatim groups    */
  uint64_t verbatim_groups;     /* V                                       */
  uint64_t stream_words;        /* W (without the 2 slack words)           */
  uint64_t code_bits;           /* sum of code lengths actually written    */
  uint64_t compressed_bytes;    /* header + sm + flags/ranks + vexp + offsets + stream */
  uint64_t export_bytes;        /* size of the UWF1 blob (sections padded to 256 B)   */
  double bits_per_weight;       /* 8 * compressed_bytes / numel            */
  int32_t has_stream;           /* Huffman stream resident                 */
  int32_t has_palette_idx;      /* 4-bit indices resident                  */
  int32_t element_bits;         /* 16: BF16 weights; 8: FP8 E4M3 weights   */
} uw_info;

const char* uw_status_str(uw_status st);
uint32_t uw_version(void);      /* (major << 16) | minor */

/* Device memory hooks.  alloc(bytes, ctx) returns device memory on the
 * current device, 256-byte aligned, or NULL; free(ptr, ctx) returns it.  */
typedef struct {
  void* (*alloc)(size_t bytes, void* ctx);
  void (*free)(void* ptr, void* ctx);
  void* ctx;
} uw_allocator;

/* Route the library's device allocations through caller hooks, e.g. a
 * framework's caching allocator: every section a handle owns, compress
 * scratch, the autotuner's buffers and uw_gemm_bf16's partial sums.  NULL (or
 * alloc == free == NULL) restores hipMalloc / hipFree.  A handle keeps the
 * hooks its sections came from and frees them through those, so the hooks
 * (and ctx) must stay valid until every handle made under them is freed.  A
 * hook returning NULL makes the allocating call fail with UW_ERR_NOMEM; a
 * block that is not 256-byte aligned is handed back and the call fails with
 * UW_ERR_INVALID.  Process-wide; UW_ERR_INVALID when exactly one hook is set.
 * (The pages state no interface; this serves the ownership rule that the
 * handle owns its compressed sections.) */
uw_status uw_set_allocator(const uw_allocator* a);

/* Destroy the HIP objects the library keeps between calls: the CU-masked
 * stream pairs and the event pool of uw_run_sequence, on every device.  It
 * synchronises those streams first.  They are made again on demand.  If never
 * called, an exit handler registered when the first of them is created
 * destroys them at exit(), before the HIP runtime's own teardown.  Must not
 * overlap a uw_run_sequence or uw_autotune call. */
uw_status uw_release_resources(void);

/* Timing aid for profilers and benchmarks.  While set, every GEMM stage call
 * that runs an MFMA kernel (the LDS-tiled and the register-fed kernels)
 * records `before` (a hipEvent_t) on the call's stream immediately before
 * its main kernel's launch and `after` immediately after it, so that the
 * elapsed time between them is that kernel alone: not the packing of x nor
 * the reduction of split-K partial sums the call may also run.  A call that
 * launches the main kernel several times (more than 64 rows on the
 * register-fed kernels) records around the first and the last launch.  Both
 * NULL clears (the default); one NULL alone is UW_ERR_INVALID.  Process-wide
 * and not synchronised with concurrent calls: for a single-threaded timing
 * loop.  It enqueues nothing by itself and changes no result. */
uw_status uw_set_kernel_events(void* before, void* after);

/* Compress a device BF16 matrix.  `w_dev` is the stored array: [n][k] for
 * UW_LAYOUT_NK, [k][n] for UW_LAYOUT_KN, given as raw 16-bit patterns.  The
 * stored row length (k for NK, n for KN) must be a multiple of 64 and the
 * element count below 2^32.  Runs the histogram, palette-membership/verbatim
 * flags, rank, segment-length and encoder kernels on `stream`; synchronises
 * the stream three times to size its allocations (tiny device-to-host
 * copies).  On success *out owns the sections.  ([EVC] "BF16權重壓縮原理") */
uw_status uw_compress(const uint16_t* w_dev, int64_t n, int64_t k, uw_layout layout,
                      const uw_compress_opts* opts, void* stream, uw_matrix** out);

/* Compress a device FP8 E4M3 matrix (OCP OFP8 E4M3: sign bit 7, exponent
 * bits 6..3, mantissa bits 2..0; any byte, NaN included, round-trips).
 * `w_dev` is the stored array of bytes, 16-byte aligned, shaped and
 * constrained as for uw_compress.  The 4-bit exponent field is coded exactly
 * as the BF16 exponent byte is (histogram, palette, code, segmented stream);
 * E4M3 has at most 16 exponent values, so every group is coded and none is
 * verbatim.  Sign and mantissa are kept as a nibble, two weights per byte
 * (numel / 2 bytes).  Allocates 2.5 x numel bytes of temporary device memory
 * and synchronises `stream` like uw_compress.  The handle serves
 * uw_decode_fp8, uw_decode_exponent (the exponent fields, one byte each),
 * uw_transcode_palette, uw_get_info, uw_sync_status and uw_free; the BF16
 * calls (uw_decode_full, uw_export, the matmul and sequence calls) return
 * UW_ERR_UNSUPPORTED.  (saidapartage.blog, "Cloudflare Unweight : -22 % sur
 * le poids de vos LLM, sans perdre un bit", section "Un complément, pas un
 * remplaçant": the coding stacks on top of quantisation.) */
uw_status uw_compress_fp8(const uint8_t* w_dev, int64_t n, int64_t k, uw_layout layout,
                          const uw_compress_opts* opts, void* stream, uw_matrix** out);

uw_status uw_get_info(const uw_matrix* m, uw_info* out);

/* Serialise to a UWF1 blob in host memory.  cap == 0 (buf may be NULL) only
 * reports the size.  Synchronises on the handle's work.  UW_ERR_STATE if the
 * Huffman stream was dropped. */
uw_status uw_export(const uw_matrix* m, void* host_buf, size_t cap, size_t* bytes);

/* Rebuild a handle from a UWF1 blob held in host memory.  The header and the
 * small sections (flags, ranks, offsets) are validated on the host before any
 * device allocation: inconsistent blobs give UW_ERR_CORRUPT.  Stream contents
 * are validated by the decoder (see uw_sync_status). */
uw_status uw_import(const void* host_blob, size_t bytes, void* stream, uw_matrix** out);

void uw_free(uw_matrix* m);

/* Full Huffman decode: writes the original stored array (numel x 16 bit) to
 * w_out_dev.  ([EVC] "四種執行管道", first pipeline) */
uw_status uw_decode_full(const uw_matrix* m, uint16_t* w_out_dev, void* stream);

/* Full decode of an FP8 handle: writes the original stored array (numel
 * E4M3 bytes, 16-byte aligned) to w_out_dev.  UW_ERR_UNSUPPORTED for a BF16
 * handle, UW_ERR_STATE once the stream was dropped; corruption is reported
 * by uw_sync_status. */
uw_status uw_decode_fp8(const uw_matrix* m, uint8_t* w_out_dev, void* stream);

/* Exponent-only decode: writes numel exponent bytes in stored order,
 * verbatim groups included.  ([EVC] "四種執行管道", second pipeline) */
uw_status uw_decode_exponent(const uw_matrix* m, uint8_t* e_out_dev, void* stream);

/* Palette transcode: numel/2 bytes; byte i holds the palette slot of element
 * 2i in its low nibble and of element 2i+1 in its high nibble; elements of
 * verbatim groups give 0.  idx_out_dev == NULL makes the indices resident in
 * the handle (direct-palette pipeline, done once at load).
 * ([EVC] "四種執行管道", third and fourth pipelines) */
uw_status uw_transcode_palette(uw_matrix* m, uint8_t* idx_out_dev, void* stream);

/* Free the Huffman stream and offsets (keeps what the direct-palette
 * pipeline needs).  Requires resident indices.  Synchronises the stream. */
uw_status uw_drop_stream(uw_matrix* m, void* stream);

/* Workspace bytes uw_matmul_reconstruct needs for pipeline p at this batch
 * (decoded BF16 / exponents / indices plus split-K partials): enough for
 * cfg == NULL (the tuned or the default kernel) and for any cfg whose
 * split_k is 0.  p may be UW_PIPE_AUTO (resolved with the current tuning
 * table; query again after changing the table).  A cfg that forces split_k
 * needs uw_workspace_size_cfg. */
uw_status uw_workspace_size(const uw_matrix* m, uw_pipeline p, int64_t batch, size_t* bytes);

/* Exactly what uw_matmul_reconstruct(m, p, ..., batch, ..., cfg) needs. */
uw_status uw_workspace_size_cfg(const uw_matrix* m, uw_pipeline p, int64_t batch, const uw_kernel_cfg* cfg,
                                size_t* bytes);

/* y[b][n] = sum_k x[b][k] * W[n][k] for b < batch, fp32 output, computed from
 * the compressed W by pipeline p.  x_dev is [batch][K] BF16 (row-major),
 * y_dev is [batch][N] fp32 (overwritten).  The workspace (device memory,
 * caller-owned, at least uw_workspace_size bytes) holds the preprocessed
 * form for pipelines 0-2.  cfg may be NULL.
 * ([EVC] "重建矩陣乘法核心運作", "四種執行管道") */
uw_status uw_matmul_reconstruct(const uw_matrix* m, uw_pipeline p, const uint16_t* x_dev,
                                int64_t batch, float* y_dev, void* ws_dev, size_t ws_bytes,
                                const uw_kernel_cfg* cfg, void* stream);

/* The GEMM stage alone, from a buffer already holding what uw_decode_full
 * (pipeline 0), uw_decode_exponent (1) or uw_transcode_palette (2) wrote for
 * this matrix; prep_dev is ignored for pipeline 3 (resident indices).  p must
 * be explicit (not UW_PIPE_AUTO).  The workspace holds only split-K partial
 * sums (of the [K][N] GEMV and of the MFMA kernels); uw_workspace_size bytes
 * are always enough for cfg == NULL or split_k == 0.  Lets a caller run the
 * preprocessing and the GEMM on different streams or at different times.
 * ([EVC] "解壓與運算資源共享": decoder and matmul are separate kernels) */
uw_status uw_matmul_stage(const uw_matrix* m, uw_pipeline p, const void* prep_dev, const uint16_t* x_dev,
                          int64_t batch, float* y_dev, void* ws_dev, size_t ws_bytes,
                          const uw_kernel_cfg* cfg, void* stream);

/* Size of the static scratch array of uw_matmul_stage_static, per GPU. */
#define UW_STATIC_SCRATCH_BYTES (64u << 20)

/* uw_matmul_stage for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and kernels, but the split-K partial sums live in a
 * static device array of UW_STATIC_SCRATCH_BYTES that each GPU the library
 * runs on holds until the process ends, instead of a caller workspace.  It
 * calls no allocating routine.  A call that would need more scratch than the
 * array holds (large batch x N with a K split) returns UW_ERR_WORKSPACE
 * before anything is enqueued: ask for fewer slices (cfg->split_k = 1 needs
 * none for the tiled kernels) or use uw_matmul_stage.  Every call on one GPU
 * shares the array: calls that overlap on one GPU (several streams or
 * threads) race and must be serialised by the caller. */
uw_status uw_matmul_stage_static(const uw_matrix* m, uw_pipeline p, const void* prep_dev, const uint16_t* x_dev,
                                 int64_t batch, float* y_dev, const uw_kernel_cfg* cfg, void* stream);

/* Several matrices with the same K sharing one x, one launch per stage where
 * the kernels allow (groups of 2 to 4): y_dev is [batch][sum of N] with matrix i's
 * columns at offset sum_{j<i} N_j.  Serves the fused gate+up projection
 * (and q+k+v): the pages tune gate and up as separate projections that read
 * the same activations ([EVC] "四種執行管道", "自動調優機制"); here they stay
 * two compressed matrices and only x and the launches are shared.
 * UW_PIPE_AUTO and cfg == NULL consult the tuning table: the group's own
 * entry first (uw_autotune_grouped), then the matrices' entries for the
 * pipeline (see uw_lookup_tuning_grouped); without an entry cfg == NULL uses
 * the grouped kernels' defaults.  Workspace: see uw_workspace_size_grouped,
 * which resolves AUTO and cfg == NULL the same way. */
uw_status uw_matmul_reconstruct_grouped(const uw_matrix* const* ms, int count, uw_pipeline p,
                                        const uint16_t* x_dev, int64_t batch, float* y_dev,
                                        void* ws_dev, size_t ws_bytes,
                                        const uw_kernel_cfg* cfg, void* stream);
uw_status uw_workspace_size_grouped(const uw_matrix* const* ms, int count, uw_pipeline p, int64_t batch,
                                    const uw_kernel_cfg* cfg, size_t* bytes);

/* Dense BF16 GEMM on an uncompressed stored array: the GEMM stage of the
 * full-decode pipeline ([EVC] "四種執行管道", first pipeline: decode to BF16,
 * then a standard matmul), also usable as a yardstick.  Partial sums of a
 * split K come from the allocator and are freed after a stream sync. */
uw_status uw_gemm_bf16(const uint16_t* w_dev, int64_t n, int64_t k, uw_layout layout,
                       const uint16_t* x_dev, int64_t batch, float* y_dev,
                       const uw_kernel_cfg* cfg, void* stream);

/* The GEMM kernel a call would run, resolved as the call resolves it
 * (UW_PIPE_AUTO, the tuning table, the default kernel table).  Introspection
 * for profiling and logs; enqueues nothing. */
typedef struct {
  int32_t pipeline;     /* resolved uw_pipeline                                  */
  int32_t variant;      /* resolved uw_kernel_cfg.variant (1..uw_variant_count) */
  int32_t fmt;          /* weights as the kernel reads them: 0 BF16, 1 exponent
                           + sign/mantissa, 2 palette, 3 palette of consecutive
                           exponents                                            */
  int32_t tile_m;       /* batch rows per block tile (0 for the GEMVs)           */
  int32_t tile_n;       /* output columns per block (per wave for the
                           register-fed kernels; 0 for the GEMVs)               */
  int32_t waves;        /* waves per block                                       */
  int32_t k_slices;     /* K split (1 = none)                                    */
  int32_t reserved;
  char kernel[64];      /* kernel name, or its prefix, as a profiler lists it   */
} uw_gemm_plan;
uw_status uw_plan_gemm(const uw_matrix* m, uw_pipeline p, int64_t batch, const uw_kernel_cfg* cfg,
                       uw_gemm_plan* out);

/* Number of GEMM variants selectable through uw_kernel_cfg.variant, numbered
 * 1..count (count = 20): 1 = VALU GEMV (v_dot2; any batch, eight rows per
 * launch); 2..10 = MFMA tiles 64x128, 128x128, 128x256, 256x128, 256x256,
 * 32x128, 32x256, 256x256 with eight waves, and 512x128 with x in registers
 * (batch rows x columns; weights rebuilt into LDS once per block, so the
 * 512-row tile rebuilds each weight once per 512 batch rows; K steps of 64);
 * 11, 12 = register-fed MFMA with two or four 16-row weight tiles per wave,
 * each wave loading its own x; 13, 14 = register-fed MFMA with one or two
 * tiles per wave, the four waves of a block sharing each window of x through
 * LDS (register-fed: weights rebuilt in registers; 64 batch rows per launch);
 * 15..20 = the MFMA tiles 64x128, 128x128, 32x128, 32x256, 512x128 with x in
 * registers and 256x128 with x in registers (eight waves of 32 rows), with
 * K steps of 128, which read whole 128-byte lines of each stored row per
 * step for twice the LDS (one block per CU).  11..20 take stored [N][K]
 * only:
 * UW_ERR_UNSUPPORTED for [K][N].  split_k applies to the KN GEMV, the
 * LDS-tiled and the register-fed MFMA kernels. */
int32_t uw_variant_count(void);

/* One entry of a sequence of projections run back to back. */
typedef struct {
  const uw_matrix* m;
  int32_t pipeline;             /* uw_pipeline                                  */
  uw_kernel_cfg cfg;
  const uint16_t* x_dev;        /* [batch][K] bf16                              */
  float* y_dev;                 /* [batch][N] fp32                              */
  int64_t batch;
} uw_job;

/* Run jobs in order.  A job's pipeline may be UW_PIPE_AUTO and a job cfg
 * whose fields are all <= 0 takes the tuned choice, as for a NULL cfg.  A
 * job's preprocessing (decode / transcode) runs on a
 * stream masked to D compute units and its GEMM on a stream masked to the
 * remaining CUs, where D is the job's cfg.decode_cus, or `decode_cus` when
 * that is 0; D = 0 runs both on `stream`.  GEMMs keep job order; the
 * workspace holds two preprocessing buffers used alternately, so
 * preprocessing runs at most one job ahead of the GEMMs and overlaps them.
 * Forks from and joins back to `stream`.  Calls that overlap on one device
 * share the library's split streams and must not run concurrently.
 * ([EVC] "解壓與運算資源共享", "跨層管道化") */
uw_status uw_sequence_workspace_size(const uw_job* jobs, int count, size_t* bytes);
uw_status uw_run_sequence(const uw_job* jobs, int count, int32_t decode_cus, void* ws_dev,
                          size_t ws_bytes, void* stream);

/* One tuned choice: for `projection` at `batch`.  n, k, layout, residency and
 * group describe the projection's matrices and key the library's tuning
 * table.  group 0: an entry for calls on one matrix (n its N).  group g in
 * 2..64: an entry for grouped calls (uw_matmul_reconstruct_grouped) on g
 * matrices that share k, layout and residency, n being their total N. */
typedef struct {
  int64_t batch;
  int32_t projection;
  int32_t pipeline;             /* uw_pipeline */
  int32_t variant;              /* uw_kernel_cfg.variant */
  int32_t split_k;
  int32_t decode_cus;
  int32_t layout;               /* uw_layout of the stored arrays            */
  int32_t residency;            /* bit 0: Huffman stream resident; bit 1:
                                   palette indices resident                  */
  int32_t group;                /* 0, or the matrix count of a grouped call  */
  uint64_t n, k;                /* logical W[N][K] shape                     */
  double sequence_us;           /* measured time of the whole tuned sequence at this batch */
} uw_tune_entry;

/* Autotuner.  ms[0..count) are the resident matrices of a model in execution
 * order, proj[i] the projection each belongs to (e.g. 0 gate, 1 up, 2 down);
 * matrices of one projection share a choice and must share shape, layout
 * and residency (UW_ERR_INVALID otherwise).  For each batch it measures
 * uw_run_sequence over all matrices, x drawn from N(0,1) in BF16, and runs
 * coordinate descent: projection 0, then 1, ..., over pipeline x GEMM
 * variant, then the K split of the chosen kernel, then the CUs of the
 * preprocessing kernel, repeating up to max_passes times until no choice
 * improves the time by 1 %.  Writes out[batch_index * nproj + projection]
 * (may be NULL) and a JSON configuration file that uw_load_tuning reads
 * (json_path may be NULL).  It does not change the library's tuning table.
 * Allocates its own x, y and workspace; synchronises `stream`.
 * ([EVC] "自動調優機制", "解壓與運算資源共享") */
uw_status uw_autotune(const uw_matrix* const* ms, const int32_t* proj, int count, int nproj,
                      const int64_t* batches, int nb, int max_passes, const char* json_path,
                      uw_tune_entry* out, void* stream);

/* Autotuner of grouped calls.  ms[0..group * ngroups) holds ngroups groups of
 * `group` matrices (2..64) in call order: group j is ms[j * group ..
 * (j + 1) * group), e.g. the gate and up matrices of successive layers.  The
 * matrices of a group share k, layout and residency (they key one table
 * entry), and every group matches the first matrix for matrix in shape,
 * layout and residency (UW_ERR_INVALID otherwise; fp8 matrices:
 * UW_ERR_UNSUPPORTED).  For each batch it measures one pass of
 * uw_matmul_reconstruct_grouped over the groups, x drawn from N(0,1) in
 * BF16, median of three timed passes after a warm-up, for every pipeline all
 * matrices can run x every GEMM variant that suits the batch (variant 0, the
 * library's rule, included), then the K split of the fastest.  Writes out[b]
 * (may be NULL) with group = `group` and n the group's total N, and a JSON
 * file in uw_autotune's format with a "group" field (json_path may be NULL).
 * It does not change the library's tuning table.  Allocates its own x, y and
 * workspace; synchronises `stream`.  ([EVC] "自動調優機制") */
uw_status uw_autotune_grouped(const uw_matrix* const* ms, int group, int ngroups, const int64_t* batches, int nb,
                              const char* json_path, uw_tune_entry* out, void* stream);

/* The tuning table that UW_PIPE_AUTO and cfg == NULL consult, keyed by
 * (n, k, layout, residency, group) with one entry per tuned batch; a call at batch B
 * takes the entry whose batch is nearest to B on a log scale (ties: the
 * smaller batch).  uw_set_tuning adds entries (an entry with the same key
 * and batch is replaced; UW_ERR_INVALID if any entry is malformed, and then
 * none is added); uw_load_tuning adds the entries of a JSON file written by
 * uw_autotune (UW_ERR_CORRUPT if it cannot be read as one, and then none is
 * added); uw_clear_tuning empties the table; uw_lookup_tuning reports the
 * entry a call on one matrix would use, uw_lookup_tuning_grouped the one a
 * grouped call on `group` matrices of total N `n` would use (UW_ERR_STATE
 * when there is none).  A grouped call with UW_PIPE_AUTO or cfg == NULL
 * takes its group entry when there is one (the pipeline, and the kernel
 * configuration when the call's pipeline is the entry's); without one, AUTO
 * takes the pipeline the matrices' own entries agree on, else direct palette
 * when every matrix has resident indices, else exponent, and cfg == NULL the
 * library's rule.  uw_load_tuning reads a missing "group" as 0.
 * Process-wide and thread safe.  ([EVC] "自動調優機制") */
uw_status uw_set_tuning(const uw_tune_entry* entries, int count);
uw_status uw_load_tuning(const char* json_path);
uw_status uw_clear_tuning(void);
uw_status uw_lookup_tuning(uint64_t n, uint64_t k, int32_t layout, int32_t residency, int64_t batch,
                           uw_tune_entry* out);
uw_status uw_lookup_tuning_grouped(uint64_t n, uint64_t k, int32_t layout, int32_t residency, int32_t group,
                                   int64_t batch, uw_tune_entry* out);

/* Free resident palette indices (keeps the Huffman form).  Synchronises. */
uw_status uw_drop_palette(uw_matrix* m, void* stream);

/* Yardsticks: the device's achievable rates, measured by the library's own
 * kernels (no compressed data involved), to read the codec and GEMM figures
 * against.  ([EVC] "GPU記憶體瓶頸成關鍵": memory bandwidth bounds inference.)
 *   kind 0: copy `bytes` (a multiple of 16) from src_dev to dst_dev with
 *           16-byte loads and stores; *work = 2 * bytes moved;
 *   kind 1: read `bytes` from src_dev; each thread stores one word of what it
 *           read to dst_dev (at most UW_YARDSTICK_SINK_BYTES); *work = bytes;
 *   kind 2: `iters` rounds of four v_mfma_f32_32x32x16_bf16 per wave on
 *           register operands, two waves per SIMD on every CU; one float per
 *           thread to dst_dev; *work = flops.
 * Pointers 16-byte aligned.  Asynchronous on `stream`. */
#define UW_YARDSTICK_SINK_BYTES (4u << 20)
uw_status uw_yardstick(int kind, const void* src_dev, void* dst_dev, size_t bytes, int64_t iters, void* stream,
                       double* work);

/* Synchronise `stream` and report whether any decoder working on m found an
 * invalid codeword or a segment whose codes overran or underran its words
 * (UW_ERR_CORRUPT); clears the flag. */
uw_status uw_sync_status(const uw_matrix* m, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UNWEIGHT_H_ */
