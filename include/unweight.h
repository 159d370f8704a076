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
  UW_PIPE_PALETTE_DIRECT = 3
} uw_pipeline;

typedef struct {
  uint32_t seg_groups;  /* groups per segment: power of two in [1, 64]; 0 = 4 */
  uint32_t flags;       /* reserved, must be 0                               */
} uw_compress_opts;

/* Kernel choice for one GEMM call.  Any field <= 0 means "library default". */
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
 * (decoded BF16 / exponents / indices plus split-K partials). */
uw_status uw_workspace_size(const uw_matrix* m, uw_pipeline p, int64_t batch, size_t* bytes);

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
 * this matrix; prep_dev is ignored for pipeline 3 (resident indices).  The
 * workspace holds only the small-batch KN kernel's partial sums; a workspace
 * of uw_workspace_size bytes is always enough.  Lets a caller run the
 * preprocessing and the GEMM on different streams or at different times.
 * ([EVC] "解壓與運算資源共享": decoder and matmul are separate kernels) */
uw_status uw_matmul_stage(const uw_matrix* m, uw_pipeline p, const void* prep_dev, const uint16_t* x_dev,
                          int64_t batch, float* y_dev, void* ws_dev, size_t ws_bytes,
                          const uw_kernel_cfg* cfg, void* stream);

/* Several matrices with the same K sharing one x (e.g. gate and up), one
 * launch per stage: y_dev is [batch][sum of N] with matrix i's columns at
 * offset sum_{j<i} N_j.  Workspace: uw_workspace_size summed over matrices. */
uw_status uw_matmul_reconstruct_grouped(const uw_matrix* const* ms, int count, uw_pipeline p,
                                        const uint16_t* x_dev, int64_t batch, float* y_dev,
                                        void* ws_dev, size_t ws_bytes,
                                        const uw_kernel_cfg* cfg, void* stream);

/* Dense BF16 GEMM on an uncompressed stored array (the GEMM stage of the
 * full-decode pipeline, also usable as a yardstick). */
uw_status uw_gemm_bf16(const uint16_t* w_dev, int64_t n, int64_t k, uw_layout layout,
                       const uint16_t* x_dev, int64_t batch, float* y_dev,
                       const uw_kernel_cfg* cfg, void* stream);

/* Number of GEMM variants selectable through uw_kernel_cfg.variant, numbered
 * 1..count: 1 = VALU GEMV (v_dot2; any batch, eight rows per launch);
 * 2..count-2 = MFMA tiles 64x128, 128x128, 128x256, 256x128, 256x256,
 * 32x128, 32x256 (batch rows x columns; weights rebuilt into LDS);
 * count-1, count = register-fed MFMA with two or four 16-row weight tiles per
 * wave (weights rebuilt in registers; 64 batch rows per launch; stored
 * [N][K] only: UW_ERR_UNSUPPORTED for [K][N]).  split_k applies to the KN
 * GEMV, the LDS-tiled and the register-fed MFMA kernels. */
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

/* Run jobs in order.  A job's preprocessing (decode / transcode) runs on a
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

/* One tuned choice: for `projection` at `batch`. */
typedef struct {
  int64_t batch;
  int32_t projection;
  int32_t pipeline;             /* uw_pipeline */
  int32_t variant;              /* uw_kernel_cfg.variant */
  int32_t split_k;
  int32_t decode_cus;
  int32_t reserved;
  double sequence_us;           /* measured time of the whole tuned sequence at this batch */
} uw_tune_entry;

/* Autotuner.  ms[0..count) are the resident matrices of a model in execution
 * order, proj[i] the projection each belongs to (e.g. 0 gate, 1 up, 2 down;
 * matrices of one projection share a choice).  For each batch it measures
 * uw_run_sequence over all matrices and runs coordinate descent: projection
 * 0, then 1, ..., over pipeline x GEMM variant, then the CUs of the
 * preprocessing kernel, repeating up to max_passes times until no choice
 * improves the time by 1 %.  Writes out[batch_index * nproj + projection]
 * (may be NULL) and a JSON configuration file (json_path may be NULL).
 * Allocates its own x, y and workspace; synchronises `stream`.
 * ([EVC] "自動調優機制", "解壓與運算資源共享") */
uw_status uw_autotune(const uw_matrix* const* ms, const int32_t* proj, int count, int nproj,
                      const int64_t* batches, int nb, int max_passes, const char* json_path,
                      uw_tune_entry* out, void* stream);

/* Free resident palette indices (keeps the Huffman form).  Synchronises. */
uw_status uw_drop_palette(uw_matrix* m, void* stream);

/* Synchronise `stream` and report whether any decoder working on m found an
 * invalid codeword or a segment whose codes overran or underran its words
 * (UW_ERR_CORRUPT); clears the flag. */
uw_status uw_sync_status(const uw_matrix* m, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UNWEIGHT_H_ */
