/*
 * nwc.h -- C ABI of libnwc: batch-1 matrix-vector products over losslessly
 * compressed BF16 (and fp8 e4m3) weights on AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the "neural-weight-compression 0.9.0"
 * PyPI page: the library holds "encoder, fused matvec, dequantization, gather"
 * ("Repository layout"); weights stay compressed and are decoded in registers
 * inside the matvec ("How it works", "Fused kernel"); dequantization and the
 * embedding lookup run on the same decoder.  The fp8 variant follows the
 * "Qwen3-4B-NWC-fp8" model card (weight-only e4m3, per-output-channel scale
 * applied at the end of the row sum, fp8 bytes recovered bit for bit).
 *
 * Conventions for every entry point:
 *  - Return value: NWC_OK (0) or a negative nwc_status.  Nothing aborts,
 *    throws, prints, allocates device memory or synchronizes the device.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check enqueues nothing.  Faults inside kernels (for example a device
 *    pointer that does not hold the blob it claims to) surface at the caller's
 *    next synchronization, not here.
 *  - "header" is a HOST pointer to the first NWC_HEADER_BYTES bytes of the
 *    blob (the caller keeps a host copy of the header; launches never read
 *    device memory on the host).  "d_blob" is the same blob in device memory.
 *  - Device work is enqueued on `stream`, a hipStream_t (NULL = the legacy
 *    default stream).  The caller owns every buffer.
 *  - Matrices are row-major: W has n rows (outputs) and k columns (inputs).
 */
#ifndef NWC_H
#define NWC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NWC_VERSION 10000 /* 1.0.0 */
#define NWC_HEADER_BYTES 256

typedef enum nwc_status {
  NWC_OK = 0,
  NWC_ERR_ARG = -1,         /* null/misaligned pointer, bad enum or flag */
  NWC_ERR_SHAPE = -2,       /* n, k, ld or a count out of range */
  NWC_ERR_CAPACITY = -3,    /* caller's buffer or workspace too small */
  NWC_ERR_FORMAT = -4,      /* header is not a valid blob of this version */
  NWC_ERR_HIP = -5,         /* the HIP runtime refused a launch */
  NWC_ERR_UNSUPPORTED = -6  /* valid request this build does not serve */
} nwc_status;

typedef enum nwc_elem {
  NWC_BF16 = 0,     /* input: uint16 BF16 bit patterns */
  NWC_FP8_E4M3 = 1  /* input: uint8 e4m3fn bytes (already quantized) */
} nwc_elem;

typedef enum nwc_coder {
  NWC_CODER_UNARY = 0,   /* the pages' code: frequency-ranked unary rank + raw
                            sign (+ raw fp8 mantissa bits), escape after 8 ranks */
  NWC_CODER_HUFFMAN = 1  /* fp8 only: length-limited (12-bit) canonical Huffman
                            code over whole fp8 bytes */
} nwc_coder;

/* Blob metadata, filled by nwc_blob_info. */
typedef struct nwc_info {
  int64_t n, k;
  int32_t elem;
  int32_t cols_per_lane;   /* C: columns of one lane's stream (one row slice) */
  int32_t rows_per_wave;   /* R: rows of a work item; 64/R lanes share a row */
  int32_t waves_per_group; /* W: work items (waves) per workgroup */
  int32_t n_spans;         /* workgroups along one row (1 unless k > 16*64*C/R) */
  int32_t n_items;         /* work items (one wave each) */
  int32_t max_rows;        /* longest item code column, in 32-bit words */
  int32_t coder;           /* nwc_coder of the blob */
  uint64_t coded_bits;     /* sum of codeword lengths of the real weights, plus
                              8 raw mantissa bits per BF16 weight */
  uint64_t total_bytes;    /* whole blob */
  uint64_t code_bytes;     /* code plane incl. per-item zero padding */
  uint64_t mant_bytes;     /* mantissa plane (0 for fp8) */
  uint64_t table_bytes;    /* header + decode table + item table */
  uint8_t rank_to_sym[128];/* frequency rank -> symbol (16 used for fp8); for
                              NWC_CODER_HUFFMAN the codeword length of byte b
                              in nibble b (low nibble of byte b/2 for even b) */
} nwc_info;

/* Library version (NWC_VERSION of the build). */
int nwc_version(void);

/* Static description of a status code. */
const char *nwc_status_string(int status);

/* Upper bound of the blob size nwc_encode can produce for an n x k matrix
 * with the same geometry request (see nwc_encode). */
int nwc_encode_bound(int64_t n, int64_t k, int elem, int cols_per_lane, int rows_per_wave, int64_t *max_bytes);

/* Host-side encoder ("How it works": byte planes, per-matrix frequency rank
 * table, unary rank code + raw sign + escape; model card: fp8 bytes coded whole).
 *   w_host   n rows of k elements, row pitch ld elements (ld >= k); uint16 BF16
 *            patterns for NWC_BF16, uint8 e4m3fn bytes for NWC_FP8_E4M3.
 *   blob     caller-owned host buffer of blob_cap bytes (see nwc_encode_bound);
 *            on success the blob occupies *blob_size bytes from its start.
 *   cols_per_lane: 0 = choose from the shape; else 16, 32, 48 or 64 columns
 *            per lane stream (a lane's decode chain is cols_per_lane/2 steps).
 *   rows_per_wave: 0 = choose from the shape; else a power of two in [1, 64]:
 *            the rows one wave decodes, each split over 64/rows_per_wave lanes.
 *            With 16 (the matrix-core geometry of nwc_matvec_batch) a
 *            workgroup gets at most 12 waves, so that two share a compute unit.
 * Any BF16 pattern (NaN payloads, infinities, zeros, subnormals) and any fp8
 * byte is encoded losslessly.  Uses up to hardware_concurrency host threads. */
int nwc_encode(const void *w_host, int64_t n, int64_t k, int64_t ld, int elem, int cols_per_lane,
               int rows_per_wave, void *blob, int64_t blob_cap, int64_t *blob_size);

/* nwc_encode with a choice of coder.  NWC_CODER_UNARY is nwc_encode.
 * NWC_CODER_HUFFMAN (fp8 only; NWC_ERR_UNSUPPORTED for BF16) is the coder
 * variant the fp8 model card's "coded whole" bytes leave room for: every fp8
 * byte of the matrix gets an optimal prefix codeword of at most 12 bits
 * (package-merge over the byte histogram), canonical order, most significant
 * bit first; byte 0x00 always has a codeword and pads the layout.  Every
 * codeword fits the decoders' 12-bit table lookup, so no code needs an
 * escape.  The device entry points decode both coders.  coder: nwc_coder;
 * other arguments and errors as nwc_encode. */
int nwc_encode_ex(const void *w_host, int64_t n, int64_t k, int64_t ld, int elem, int coder, int cols_per_lane,
                  int rows_per_wave, void *blob, int64_t blob_cap, int64_t *blob_size);

/* Validate a blob header (host pointer, at least NWC_HEADER_BYTES) and
 * describe it.  blob_bytes: bytes available at `blob` (>= header bytes). */
int nwc_blob_info(const void *blob, int64_t blob_bytes, nwc_info *info);

/* Full validation of a blob in host memory (blob_bytes available at `blob`),
 * for blobs read from storage: the header as nwc_blob_info checks it, the
 * rank table (each symbol once), the decode table (equal to the one the rank
 * table defines: "How it works", frequency-ranked unary code), and the item
 * table (every item's code rows inside the code plane, 1..max_rows whole
 * 256-byte rows).  The device entry points trust the item table, whose
 * offsets bound their memory accesses: check a blob that did not come from
 * nwc_encode in this process before uploading it.  Reads only; O(blob
 * header + tables).  NWC_ERR_CAPACITY if blob_bytes is shorter than the blob,
 * NWC_ERR_FORMAT for any inconsistency. */
int nwc_blob_check(const void *blob, int64_t blob_bytes);

/* Device workspace bytes nwc_matvec needs for this blob: 0 unless a row is
 * split over several workgroups (n_spans > 1, only for k > 16*64*C/R), then
 * fp32 partial sums of each row per span.  Its contents need no
 * initialisation and are overwritten by every call. */
int nwc_workspace_size(const void *header, int64_t *bytes);

/* Fused decode + matvec ("Fused kernel": weights decoded in registers, fp32
 * row sums; model card: fp8 scale applied after the row sum).
 *   d_x      device, k BF16 patterns (uint16), 16-byte aligned.
 *   d_scale  device, n fp32 scales for NWC_FP8_E4M3 blobs; must be NULL for BF16.
 *   d_y      device, n fp32 outputs, 4-byte aligned:  y_i = (s_i *) sum_j w_ij x_j.
 *   d_ws     device workspace of ws_bytes >= nwc_workspace_size, 256-byte
 *            aligned; may be NULL when the size is 0.  Concurrent calls need
 *            distinct workspaces.
 * One kernel: a workgroup decodes whole rows and sums them across its lanes
 * and waves.  Only when n_spans > 1 is a second small kernel enqueued to sum
 * the spans' partials.  The summation order is fixed, so repeated calls give
 * identical bits. */
int nwc_matvec(const void *header, const void *d_blob, const void *d_x, const float *d_scale,
               float *d_y, void *d_ws, int64_t ws_bytes, void *stream);

/* nwc_matvec for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and the same bits as nwc_matvec, with no workspace argument.
 * Matrices whose rows span several workgroups (nwc_workspace_size > 0) keep
 * their fp32 span partials in a static device array of the library,
 * NWC_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on a GPU until
 * the process ends; a matrix needing more is refused (NWC_ERR_CAPACITY, with
 * nothing enqueued).  Nothing is allocated and nothing needs clearing (every
 * partial is written before it is read).  All calls on one GPU share its
 * array: calls that may overlap in time on one GPU (different streams, or
 * several threads) race on it and must be serialized by the caller; calls on
 * one stream are ordered.  Other arguments and errors as nwc_matvec. */
#define NWC_NOALLOC_SCRATCH_BYTES (4u << 20)
int nwc_matvec_noalloc(const void *header, const void *d_blob, const void *d_x, const float *d_scale, float *d_y,
                       void *stream);

/* Several fused decode + matvec products in one launch: y_m = W_m x_m (times
 * the fp8 row scales) for m < count, each matrix with its own activation and
 * output.  This is the library's form of the pages' projection fusion ("Install"
 * usage and "Run a model" on the PyPI page: projections that read the same
 * input, such as q, k and v, or gate and up, run together): the matrices stay
 * separately encoded, each with its own rank table, and share one kernel
 * launch -- pass the same d_x for projections of one input.
 *   mats     host array of count descriptors, each as the arguments of
 *            nwc_matvec (host header copy, device blob, activation, fp8 scales
 *            or NULL, output); 1 <= count <= NWC_GROUP_MAX (0 does nothing).
 * Matrices of one work-item shape (element type, columns per lane, rows per
 * wave, waves per workgroup) share a launch; a group of several shapes is one
 * launch per shape, in order of first appearance (inside a launch the
 * workgroups take the matrices smallest first).  Every output is bit-equal
 * to nwc_matvec on the same matrix and activation.  Matrices whose rows span
 * several workgroups (n_spans > 1) need a workspace and are refused
 * (NWC_ERR_UNSUPPORTED).  Outputs must not overlap each other or any input.
 * Every descriptor is checked before anything is enqueued. */
#define NWC_GROUP_MAX 12
typedef struct nwc_matvec_desc {
  const void *header;
  const void *d_blob;
  const void *d_x;
  const float *d_scale;
  float *d_y;
} nwc_matvec_desc;
int nwc_matvec_group(const nwc_matvec_desc *mats, int count, void *stream);

/* Fused decode + matvec for a small batch of activation rows (the pages'
 * batch-1 "token path" widened to a few tokens; "Fused kernel" and
 * "Limitations" describe batch 1 and the prefill route, a batch of several
 * rows is this library's addition): y_b = W x_b for b < batch.
 *   d_x      device, batch rows of k BF16 patterns, row b at d_x + b*ldx
 *            elements; ldx >= k and a multiple of 8 (16-byte aligned rows).
 *   d_y      device, batch rows of n fp32, row b at d_y + b*ldy; ldy >= n.
 *   d_scale, d_ws, ws_bytes: as nwc_matvec (rows share the workspace in turn).
 * BF16 blobs encoded with 16 rows per wave and 16 or 32 columns per lane
 * (nwc_encode with rows_per_wave = 16), for 5 rows or more and ldx < 2^25:
 * the matrix-core path (the pages' planned tensor-core accumulation, "Status
 * and limitations"): every weight is decoded once per 32 activation rows and
 * the products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; each
 * output is within the matvec tolerance of the exact sum (the summation
 * order differs from nwc_matvec but is fixed: repeated calls give the same
 * bits), activations past column k are never used, and the workspace is not
 * used.
 * Other BF16 blobs with one span per row and at most 32 columns per lane
 * decode every weight once per group of up to four rows, each row summed in
 * the same order as nwc_matvec, so row b equals nwc_matvec on x_b bit for
 * bit; other blobs run one row at a time.  batch == 0 does nothing. */
int nwc_matvec_batch(const void *header, const void *d_blob, const void *d_x, int64_t ldx, int64_t batch,
                     const float *d_scale, float *d_y, int64_t ldy, void *d_ws, int64_t ws_bytes, void *stream);

/* Dequantization to the stored element type ("How it works": dequantization
 * runs on the same decoder).  BF16 blobs write uint16 BF16 patterns, fp8 blobs
 * write the fp8 bytes (the scale is not applied).  Row i of the matrix goes to
 * d_w + i*ld elements (ld >= k); d_w 16-byte aligned. Bit-exact. */
int nwc_dequant(const void *header, const void *d_blob, void *d_w, int64_t ld, void *stream);

/* Embedding lookup on the same decoder ("How it works": tied lm_head and
 * embedding share one encoding).  For t < n_ids, row d_ids[t] is decoded to
 * d_out + t*k elements (BF16 patterns or fp8 bytes).  Ids outside [0, n)
 * produce a zero row.  d_ids: device int64; bit-exact. */
int nwc_gather(const void *header, const void *d_blob, const int64_t *d_ids, int64_t n_ids,
               void *d_out, void *stream);

/* Measurement helper, not part of the method: a plain streaming read of
 * `bytes` (a multiple of 16) at d_buf (device, 16-byte aligned) with 16-byte
 * loads, the achievable-bandwidth reference the matvec is compared with.
 * d_sink: device, one uint32 the kernel may write (practically never does). */
int nwc_stream_read(const void *d_buf, int64_t bytes, uint32_t *d_sink, void *stream);

/* Measurement helper, not part of the method: the uncompressed baseline, a
 * plain BF16 GEMV y = W x with fp32 accumulation and no decode (one wave per
 * row streaming 16-byte chunks of the row and of x).
 *   d_w  device, n rows of BF16 patterns, row pitch ldw elements (ldw >= k,
 *        a multiple of 8), 16-byte aligned.
 *   d_x  device, k BF16 patterns, 16-byte aligned; k >= 8, a multiple of 8.
 *   d_y  device, n fp32 outputs, 4-byte aligned.
 * NWC_ERR_ARG for null or misaligned pointers, NWC_ERR_SHAPE otherwise. */
int nwc_bf16_gemv(const void *d_w, int64_t n, int64_t k, int64_t ldw, const void *d_x, float *d_y, void *stream);

/* Measurement helper: several plain BF16 GEMVs in one launch (the launch
 * structure of nwc_matvec_group), each described as the arguments of
 * nwc_bf16_gemv; 1 <= count <= NWC_GROUP_MAX (0 does nothing).  Every
 * descriptor is checked before anything is enqueued. */
typedef struct nwc_bf16_gemv_desc {
  const void *d_w;
  int64_t n, k, ldw;
  const void *d_x;
  float *d_y;
} nwc_bf16_gemv_desc;
int nwc_bf16_gemv_group(const nwc_bf16_gemv_desc *mats, int count, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* NWC_H */
