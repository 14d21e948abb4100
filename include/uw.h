/*
 * uw.h -- C ABI of libuw: lossless BF16 weight compression fused into the decode-time GEMM,
 * for AMD MI355X (gfx950).
 *
 * Method: Cloudflare blog post "Unweight" (unweight-tensor-compression).
 *  - BF16 anatomy paragraph: a BF16 weight is sign | 8-bit exponent | 7-bit mantissa; sign and
 *    mantissa are stored unchanged (one "sm" byte per weight).
 *  - Exponent-distribution paragraph and figure: the 16 most frequent exponents of a matrix
 *    (its palette) cover more than 99 % of its weights.
 *  - Huffman paragraph: the exponent alone is Huffman coded.
 *  - Rare-exponent paragraph: a run of 64 weights of one row that holds an exponent outside
 *    the palette is kept verbatim, so the hot path decides once per run, not per element.
 *  - Four-pipeline paragraphs: full Huffman decode then a standard GEMM; exponent-only decode;
 *    run-time transcode to 4-bit palette indices; direct palette (indices prepared at model
 *    load, no per-step preprocessing).  The last three feed a matmul that rebuilds BF16 on
 *    chip, so the rebuilt matrix never goes through HBM.
 *  - Autotuning paragraphs: the pipeline is chosen per weight matrix and batch size by
 *    measurement.
 *
 * Conventions (all entry points):
 *  - Every function returns uw_status (0 = UW_OK); on failure uw_last_error() returns a message
 *    (thread-local, valid until the next call on the same thread).
 *  - All pointers are borrowed; the caller owns every buffer.  The library never allocates
 *    device memory and keeps no device state.
 *  - Host validation happens before any launch: a call that returns an error launched nothing.
 *  - Device calls are asynchronous on the given stream and report launch errors only; data
 *    errors found by a kernel (a corrupt bitstream) are recorded in the workspace's error word
 *    and reported by uw_check().
 *  - Shapes: W is [n, k] BF16 row-major (output x input, like a Linear weight), X is [m, k]
 *    BF16 row-major, Y = X W^T is [m, n] fp32 row-major.  k must be a multiple of 64.
 *
 * Storage format "UW1" (little-endian; a reading of the post where it is silent):
 *   Rows are grouped in tiles of 16 (np = n rounded up to 16, T = np/16 tiles); columns in
 *   blocks of 64 (KB = k/64).  A segment is (tile t, block b, row r): 64 weights of row 16t+r.
 *   Segments are enumerated in (t, b, r) order.
 *   - palette: the min(16, #distinct) exponents with the highest whole-matrix counts (ties to the
 *     smaller exponent), listed in ascending order; the palette index is the list position.
 *   - sm:      np*k bytes, sign<<7 | mantissa, in 16x16 sub-tiles: byte (row, col) sits at
 *              ((t*(k/16) + col/16)*16 + row%16)*16 + col%16.
 *   - flags:   T*KB uint16; bit r of flags[t*KB + b] = segment (t, b, r) is verbatim.
 *   - vprefix: T+1 uint32; verbatim segments in tiles before t.
 *   - vexp:    64 raw exponent bytes per verbatim segment, in segment order.
 *   - words:   Huffman stream of the palette indices of every non-verbatim segment (segment
 *              order, column ascending), codes MSB-first in uint32 words, two zero words after.
 *              Code: canonical prefix code, at most 13 bits a code (the format's limit);
 *              uw_encode writes the optimal code limited to 12 bits (lmax = 12 in the header),
 *              so that every code fits the decoders' 2^12-entry, 16 KB lookup table.
 *   - off:     uint32 start bit of every chunk, then the total bit count.  A chunk is at most
 *              `chunk` coded symbols (a multiple of 64); chunks restart at every 64-column
 *              block of every tile, so block b of a tile holds ceil(64*coded rows/chunk).
 *   - cbase:   T+1 uint32; first chunk of every tile.
 *   Direct-palette index stream (made by uw_transcode_palette, held by the caller): np*k/2 bytes;
 *   row r of sub-tile (t, j) owns 8 bytes at ((t*(k/16) + j)*16 + r)*8 = two uint32 words, word w
 *   holding columns 16j+8w+i (i = 0..7) at bit 4*(i/2) + 16*(i%2); verbatim segments and
 *   padding rows hold 0.
 */
#ifndef UW_H
#define UW_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t uw_status;
enum {
  UW_OK = 0,
  UW_E_ARG = -1,       /* null pointer, bad enum, non-positive size */
  UW_E_SHAPE = -2,     /* k % 64 != 0, m outside [1, UW_MAX_M], size limits */
  UW_E_FORMAT = -3,    /* blob: bad magic/version/geometry, section bounds, inconsistent tables */
  UW_E_NOMEM = -4,     /* host allocation failed */
  UW_E_WORKSPACE = -5, /* workspace missing or too small */
  UW_E_HIP = -6,       /* HIP launch or runtime error */
  UW_E_DATA = -7       /* a kernel found a corrupt stream (reported by uw_check) */
};
enum {
  UW_PIPE_AUTO = 0,           /* autotune table entry for (n, k, m), else DIRECT_PALETTE */
  UW_PIPE_FULL_DECODE = 1,    /* Huffman -> BF16 W in workspace, then BF16 GEMM */
  UW_PIPE_EXP_ONLY = 2,       /* Huffman -> exponent bytes in workspace, then sm+exp GEMM */
  UW_PIPE_TRANSCODE = 3,      /* Huffman -> 4-bit indices in workspace, then palette GEMM */
  UW_PIPE_DIRECT_PALETTE = 4, /* resident 4-bit indices (bound at uw_dmat_bind), palette GEMM */
  UW_PIPE_BF16 = 5            /* autotune key of the uncompressed uw_gemm_bf16 (not a uw_gemm pipeline) */
};
#define UW_MAX_M 1024
#define UW_MAX_CHUNK 4096

/* Message for the last failing call on this thread ("" if none). */
const char* uw_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int32_t uw_version(void);

/* ------------------------------------------------------------------------------------------
 * Host encoder (pure, thread-safe, host pointers only).
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  uint32_t n;               /* palette size, 1..16 */
  uint8_t exp[16];          /* palette exponents, ascending; exp[i] for i >= n is 0 */
  uint8_t index_of[256];    /* exponent -> palette index, 0xFF when outside the palette */
  uint64_t hist[256];       /* whole-matrix exponent histogram */
} uw_palette;

/* Histogram and top-16 palette of W (exponent-distribution paragraph).
 * w: host, n*k uint16 BF16 bit patterns, row-major.  Errors: UW_E_ARG, UW_E_SHAPE. */
uw_status uw_build_palette(const uint16_t* w, int64_t n, int64_t k, uw_palette* out);

/* Upper bound of the blob size for an n x k matrix (every segment coded at 13 bits). */
uw_status uw_encode_bound(int64_t n, int64_t k, int32_t chunk, size_t* bytes);

/* Encode W into a UW1 blob (Huffman, rare-exponent and four-pipeline paragraphs).
 * w:      host, n*k BF16 bit patterns, row-major.
 * p:      the palette to encode with, or NULL to build W's own (uw_build_palette's choice).
 *         A caller palette (e.g. one shared by several matrices, or another matrix's) replaces
 *         only that step: every 64-weight segment holding an exponent outside it is stored
 *         verbatim and the Huffman code is built over the indices of the other segments.
 *         Checked: 1 <= n <= 16, exp[0..n-1] strictly ascending, index_of[exp[i]] == i and
 *         0xFF for every other exponent (UW_E_ARG otherwise); hist is not read.
 * chunk:  coded symbols per chunk, a multiple of 64 in [64, UW_MAX_CHUNK]; 0 = 512 (a block
 *         holds at most 1024 coded symbols, so values above 1024 act as 1024).
 * blob:   host output of `cap` bytes; NULL asks for the exact size only (two-call pattern).
 * used:   receives the blob size in bytes.
 * Errors: UW_E_ARG (null w/used, bad palette), UW_E_SHAPE (k % 64, stream >= 2^32 bits),
 *         UW_E_NOMEM, UW_E_WORKSPACE (cap too small; *used holds the size needed). */
uw_status uw_encode(const uint16_t* w, int64_t n, int64_t k, const uw_palette* p, int32_t chunk,
                    void* blob, size_t cap, size_t* used);

/* Header fields of a blob, validated (host).  Sizes in bytes. */
typedef struct {
  int64_t n, k, np, tiles, kb;
  int32_t chunk, lmax, n_pal, affine;      /* affine: palette[i] == palette[0] + i for all i */
  int64_t n_verb, n_coded, total_bits, n_chunks, n_words;
  uint8_t palette[16];
  uint8_t code_len[16];
  uint16_t code[16];
  uint64_t sec_off[7], sec_size[7];         /* sm, flags, vprefix, vexp, cbase, off, words */
  uint64_t blob_bytes;                      /* header + sections, as laid out */
  uint64_t resident_bytes;                  /* sm + idx + flags + vprefix + vexp */
  uint64_t idx_bytes;                       /* np*k/2, the direct-palette index stream */
} uw_info;
uw_status uw_blob_info(const void* blob_host, size_t bytes, uw_info* out);

/* ------------------------------------------------------------------------------------------
 * Device view of an encoded matrix.
 * ------------------------------------------------------------------------------------------ */
typedef struct uw_dmat uw_dmat;  /* opaque; the caller allocates uw_dmat_size() bytes */
size_t uw_dmat_size(void);

/* Validate the blob (host copy) and record the device addresses of its sections.
 * blob_host: host copy of the blob (read during the call only); bytes: its size.
 * blob_dev:  device copy of the same bytes (must stay valid while d is used).
 * idx_dev:   device buffer of uw_info.idx_bytes for the direct-palette index stream, or NULL
 *            (then UW_PIPE_DIRECT_PALETTE is refused with UW_E_ARG).
 * With a current device, the call also builds the Huffman decoder's 16 KB lookup table for the
 * blob's code lengths and copies it (synchronously, once per distinct code) into a fixed
 * per-device table cache of 128 codes; decode calls on that device then load the table instead
 * of building it in every workgroup.  Without a device, with a full cache, on another device or
 * with UW_ROW_TABLE_IN_KERNEL set in the environment, the decoder builds the table itself
 * (same results).  A failed copy is not an error.
 * Errors: UW_E_ARG, UW_E_FORMAT. */
uw_status uw_dmat_bind(uw_dmat* d, const void* blob_host, size_t bytes, const void* blob_dev,
                       void* idx_dev);
uw_status uw_dmat_get_info(const uw_dmat* d, uw_info* out);

/* Workspace bytes a call needs.  op: a UW_PIPE_* value for uw_gemm, or one of the decode
 * targets below.  Layout: [256 bytes: error word][decoded matrix, decode pipelines only]
 * [fp32 K-slice partial sums of the multi-tile and wide-tile kernels: up to 16 slices of m x n,
 *  fewer at large m].
 * The first 256 bytes must be zero before the first use (uw_check clears the word again); the
 * rest needs no initialisation.  One workspace may serve any sequence of calls (any matrix, m,
 * pipeline) issued in order on one stream; calls that may overlap need workspaces of their own.
 * The partial-sum room is optional: uw_gemm uses as many K slices as the room it is given holds
 * (none with ws NULL or only the error word), which changes speed and the fp32 summation order
 * (results stay within the GEMM tolerance; the same room gives bit-identical results). */
enum { UW_OP_DECODE_FULL = 16, UW_OP_TRANSCODE = 17, UW_OP_DECODE_EXP = 18 };
uw_status uw_workspace_size(const uw_dmat* d, int32_t m, int32_t op, size_t* bytes);

/* Full Huffman decode (pipeline 1's preprocessing): w_out (device, n*k uint16, row-major) is
 * bit-identical to the encoded W.  ws: workspace of uw_workspace_size(.., UW_OP_DECODE_FULL).
 * The three decode entry points write intermediate data into their output buffer before its
 * final contents (decoded index words, in decode order), so the output must not alias an input
 * and must not be read until the call has completed on its stream. */
uw_status uw_decode_full(const uw_dmat* d, uint16_t* w_out, void* ws, size_t ws_bytes,
                         hipStream_t s);

/* Huffman -> 4-bit palette index stream (pipeline 3's preprocessing, and the load-time
 * transcode of the direct-palette format): idx_out (device, uw_info.idx_bytes). */
uw_status uw_transcode_palette(const uw_dmat* d, uint8_t* idx_out, void* ws, size_t ws_bytes,
                               hipStream_t s);

/* Huffman -> exponent bytes (pipeline 2's preprocessing): exp_out (device, np*k bytes, the sm
 * sub-tile layout; verbatim segments get their raw exponents, padding rows 0). */
uw_status uw_decode_exponents(const uw_dmat* d, uint8_t* exp_out, void* ws, size_t ws_bytes,
                              hipStream_t s);

/* Y = X W^T with W rebuilt on chip (reconstructive-matmul paragraphs).
 * x: device [m, k] BF16; y: device [m, n] fp32; 1 <= m <= UW_MAX_M.
 * pipeline: UW_PIPE_AUTO..UW_PIPE_DIRECT_PALETTE; variant: kernel variant id (uw_variant_count),
 * -1 = the autotune table's variant for (n, k, m, pipeline), else the built-in default.
 * ws: workspace of uw_workspace_size(d, m, pipeline) bytes.  The direct-palette pipeline also
 * accepts NULL or less (fewer K slices, see uw_workspace_size); the decode pipelines need at
 * least the error word and their decoded matrix, else UW_E_WORKSPACE.
 * Errors: UW_E_ARG, UW_E_SHAPE, UW_E_WORKSPACE, UW_E_HIP. */
uw_status uw_gemm(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t pipeline,
                  void* ws, size_t ws_bytes, hipStream_t s);
uw_status uw_gemm_variant(const uw_dmat* d, const uint16_t* x, float* y, int32_t m,
                          int32_t pipeline, int32_t variant, void* ws, size_t ws_bytes,
                          hipStream_t s);

/* Allocation-free form of uw_gemm_variant(d, x, y, m, UW_PIPE_DIRECT_PALETTE, variant, ws, ...),
 * for callers that cannot allocate device memory around the call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace argument, and the call
 * allocates nothing.  The K-slice partial sums of the multi-tile and wide-tile kernels go to a
 * device array inside the library of 64 MiB per GPU (held on every GPU the library runs on until
 * the process ends).  With the same variant the result is bit-identical to uw_gemm_variant given
 * a workspace of uw_workspace_size(d, m, UW_PIPE_DIRECT_PALETTE) bytes.  The array is shared by
 * every call on a GPU: calls that may overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  x, y, m, variant and stream as uw_gemm_variant; d needs an
 * index stream bound.  Errors: UW_E_ARG, UW_E_SHAPE, UW_E_HIP, and UW_E_WORKSPACE when the
 * call's partial sums (uw_workspace_size(...) - 256 bytes) exceed 64 MiB; nothing is launched
 * on an error. */
uw_status uw_gemm_noalloc(const uw_dmat* d, const uint16_t* x, float* y, int32_t m, int32_t variant,
                          hipStream_t s);

/* Uncompressed baseline (the BF16 GEMM of pipeline 1): Y = X W^T for a plain BF16 W
 * (device, [n, k] row-major).  variant: -1 = the UW_PIPE_BF16 autotune entry, else default. */
uw_status uw_gemm_bf16(const uint16_t* w, int64_t n, int64_t k, const uint16_t* x, float* y,
                       int32_t m, int32_t variant, hipStream_t s);

/* Kernel variants: count, and a description string of one: "waves=W unroll=U" (per-tile
 * kernel), "multitile tiles=W unroll=U", "shared-x tiles=W unroll=U" (M <= 16),
 * "wide pairs=W unroll=U", "big tile=NxM" or "big tile=NxM waves=8" (large batches, palette
 * sources; others run the default multi-tile variant).  Every variant computes any shape and batch size the entry
 * points accept; a variant whose conditions a call does not meet runs a default instead. */
int32_t uw_variant_count(void);
const char* uw_variant_name(int32_t variant);

/* Wait for s and report a data error recorded in ws (UW_E_DATA), clearing it. */
uw_status uw_check(void* ws, hipStream_t s);

/* Autotune table (autotuning paragraphs: the pipeline and kernel are chosen per weight shape
 * and batch size by measurement).  Two kinds of entry, keyed by (n, k, m):
 *  - the pipeline UW_PIPE_AUTO runs, with its variant (uw_autotune_set; it also records that
 *    variant for that pipeline);
 *  - the variant a concrete pipeline, or UW_PIPE_BF16 for uw_gemm_bf16, runs with when called
 *    with variant -1 (uw_autotune_set_variant; variant -1 deletes the entry).
 * Lookup (dispatch and the getters alike): the (n, k, m) entry; else the entry of the nearest
 * measured batch size for the same (n, k) -- nearest by ratio m'/m, the smaller m' on a tie --
 * so a table measured at a few M also serves the sizes between; else, with no entry for
 * (n, k) at all, AUTO runs DIRECT_PALETTE and variant -1 takes the built-in default.
 * Text file for uw_autotune_load, one entry per line, '#' starts a comment:
 *     n k m pipeline variant             (AUTO entry)
 *     variant n k m pipeline variant     (per-pipeline variant)
 * The file is parsed and checked whole before any entry is applied (UW_E_ARG on a bad line).
 * The table is process-wide and guarded by a mutex. */
uw_status uw_autotune_load(const char* path);
uw_status uw_autotune_set(int64_t n, int64_t k, int32_t m, int32_t pipeline, int32_t variant);
uw_status uw_autotune_get(int64_t n, int64_t k, int32_t m, int32_t* pipeline, int32_t* variant);
uw_status uw_autotune_set_variant(int64_t n, int64_t k, int32_t m, int32_t pipeline,
                                  int32_t variant);
uw_status uw_autotune_get_variant(int64_t n, int64_t k, int32_t m, int32_t pipeline,
                                  int32_t* variant);
uw_status uw_autotune_clear(void);

/* Glue of an MLP decode step (SwiGLU between up/gate and down):
 * h[i] = bf16(silu(g[i]) * u[i]) in fp32, round to nearest even; count elements. */
uw_status uw_swiglu(const float* g, const float* u, uint16_t* h, int64_t count, hipStream_t s);

/* The up projection with the SwiGLU glue fused into its output: h = bf16(silu(gate) * (x W^T))
 * element by element ([m, n]; W = the bound matrix, typically up_proj; gate = the fp32 output
 * of the gate projection, e.g. from uw_gemm earlier on the same stream).  The GEMM is exactly
 * uw_gemm_variant's (same kernels, same summation order) and the epilogue the arithmetic of
 * uw_swiglu, so h equals uw_gemm_variant followed by uw_swiglu bit for bit, without the fp32
 * product going through memory.  gate: device fp32 [m, n], 16-byte aligned; h: device BF16
 * bits [m, n], 8-byte aligned.  Other arguments, workspace and errors as uw_gemm_variant. */
uw_status uw_gemm_swiglu(const uw_dmat* d, const uint16_t* x, const float* gate, uint16_t* h,
                         int32_t m, int32_t pipeline, int32_t variant, void* ws, size_t ws_bytes,
                         hipStream_t s);
/* x[r, :] = bf16(y[r, :] / sqrt(mean(y[r, :]^2) + eps)) for rows r < m of an [m, n] fp32 y. */
uw_status uw_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps,
                     hipStream_t s);

/* The down projection with the RMS norm fused after it: y = x W^T (fp32 [m, n], as uw_gemm_variant)
 * and xn[r, :] = bf16(y[r, :] / sqrt(mean(y[r, :]^2) + eps)) (BF16 bits [m, n]), equal bit for bit
 * to uw_gemm_variant followed by uw_rmsnorm.  When the call runs the multi-tile kernel with K
 * slices (workspace room for them), the norm is computed inside the slice reduction, one launch
 * fewer; otherwise it runs as a separate pass over y.  Arguments, workspace and errors as
 * uw_gemm_variant; xn: device, [m, n]. */
uw_status uw_gemm_rmsnorm(const uw_dmat* d, const uint16_t* x, float* y, uint16_t* xn, int32_t m,
                          float eps, int32_t pipeline, int32_t variant, void* ws, size_t ws_bytes,
                          hipStream_t s);

/* Hard/easy MLP decode step (hard/easy-layer paragraphs of the post: a "hard" layer keeps only
 * its Huffman bundle resident and is decoded ahead of use, off the critical path, while the GPU
 * computes the layers before it; an "easy" layer is held in the direct-palette form).
 *
 * A step runs `layers` layers of the MLP stack (gate, up: [inter, hidden]; down: [hidden, inter]):
 *   g = x gate^T; h = bf16(silu(g) * (x up^T)) (uw_gemm_swiglu); y = h down^T and
 *   x' = bf16(y / sqrt(mean(y^2) + eps)) (uw_gemm_rmsnorm) -- the same calls, kernels and bits as
 * issuing those entry points one by one with UW_PIPE_DIRECT_PALETTE and the autotuned variant.
 * Matrix j of layer l is mats[3l + j] (j = 0 gate, 1 up, 2 down).  hard[3l + j] != 0: the view's
 * own index stream is not used (it may be unbound); its 4-bit index stream is decoded on `side`
 * into one of two slot sets (hard layers alternate between them) while `main` runs the layers
 * before it, with events ordering decode -> use -> reuse.  Easy matrices need an index stream
 * bound at uw_dmat_bind.  At most two hard layers are decoded ahead.
 *
 * Caller-owned device buffers (borrowed until uw_sched_release):
 *   slots     2 * 3 * slot_bytes; slot_bytes >= idx_bytes of every hard matrix (uw_info)
 *   g         m * inter fp32 (16-byte aligned);  h  m * inter BF16 (8-byte aligned)
 *   y         m * hidden fp32;  xo  2 * m * hidden BF16: the two ping-pong layer outputs
 *   ws        main-stream workspace: at least uw_workspace_size(m, UW_PIPE_DIRECT_PALETTE) of
 *             every matrix (K-slice partial sums; may be NULL: no K split)
 *   dws       side-stream error word, >= 256 bytes, zeroed; uw_check(dws) reports a corrupt
 *             bitstream found by a decode
 * The scheduler holds host state and four HIP events (no device memory): the caller allocates
 * uw_sched_size() bytes for it and ends its use with uw_sched_release.  Errors: UW_E_ARG (null
 * pointer, bad shape or stream), UW_E_SHAPE (a matrix not of its layer shape, m outside
 * [1, UW_MAX_M]), UW_E_WORKSPACE (slot_bytes or a buffer too small), UW_E_NOMEM, UW_E_HIP; on an
 * error nothing was launched. */
typedef struct uw_sched uw_sched;
size_t uw_sched_size(void);
uw_status uw_sched_init(uw_sched* s, int32_t layers, int32_t m, int32_t hidden, int32_t inter,
                        const uw_dmat* const* mats, const uint8_t* hard, void* slots,
                        size_t slot_bytes, float* g, uint16_t* h, float* y, uint16_t* xo,
                        void* ws, size_t ws_bytes, void* dws, size_t dws_bytes, float eps,
                        hipStream_t main_stream, hipStream_t side_stream);
/* One step from x (device BF16 [m, hidden]); *out receives the device address of the last
 * layer's output (one of the two halves of xo).  Asynchronous on the main stream; the side
 * stream's decodes are ordered by events, and the next step's first decodes wait for this
 * step's last use of their slots. */
uw_status uw_sched_step(uw_sched* s, const uint16_t* x, uint16_t** out);
/* Per-layer record of every following step (for checking each GEMM of a scheduled step on its
 * own inputs): after layer l's GEMMs the main stream copies g [m, inter] fp32, h [m, inter] BF16,
 * y [m, hidden] fp32 and the layer output [m, hidden] BF16, back to back, to
 * trace + l * m * (6 * inter + 6 * hidden).  trace: device, at least layers times that many
 * bytes (UW_E_WORKSPACE otherwise), borrowed until replaced; NULL stops the recording. */
uw_status uw_sched_trace(uw_sched* s, void* trace, size_t bytes);
/* Decode/GEMM split of the chip (SM-split paragraph of the post: the decoder and the matmul run
 * on separate parts of the GPU, and the split is tuned).  decode_workgroups > 0: each hard-layer
 * decode runs on at most that many decoder workgroups, which take the matrix's decode units in
 * turn (the table is built once per workgroup); a workgroup of the decoder fills the LDS of a
 * compute unit, so this is the number of compute units the decodes occupy while the main
 * stream's GEMMs run on the others.  0 (the default): the whole chip.  Results do not depend on
 * it.  Errors: UW_E_ARG. */
uw_status uw_sched_split(uw_sched* s, int32_t decode_workgroups);
/* Releases the events and host state (waits for nothing: the caller synchronises first). */
uw_status uw_sched_release(uw_sched* s);

#ifdef __cplusplus
}
#endif
#endif /* UW_H */
