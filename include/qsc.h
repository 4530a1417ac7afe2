/*
 * qsc — ANS-resident 4D-STEM detector counts with fused decode + virtual
 * detector reductions on AMD Instinct MI355X (gfx950).
 *
 * Counts I[s, p] (scan s in row-major order, detector pixel p = kr*det_cols +
 * kc, native uint8 or uint16) stay entropy coded in device memory as the
 * container defined in FORMAT.md (byte-rANS or paired tANS layout, 512-scan
 * blocks, per-pixel streams, grouped offsets). Queries decode and reduce in one
 * pass on the GPU.
 *
 * Conventions for every entry point:
 *  - Return value: QSC_OK (0) or a negative qsc_status.
 *  - "host" pointers are CPU memory, "device" pointers are HIP device memory
 *    of the resident's GPU. The caller owns every buffer it passes in; the
 *    library owns the resident and everything it allocates for it.
 *  - hip_stream is a hipStream_t (NULL = the default stream). Queries are
 *    enqueued on it. With wait = 0 a query only enqueues and its decode status
 *    is reported by qsc_finish; with wait = 1 it synchronises the stream and
 *    returns QSC_ERR_MALFORMED if any stream it decoded was malformed, in
 *    which case the output buffer holds no result (paired-resident page,
 *    "Contract": a malformed stream fails the query and no result is
 *    returned).
 *  - Argument errors are detected on the host before anything is enqueued and
 *    leave outputs untouched.
 *  - Calls that enqueue work on the same resident must not run concurrently
 *    from several host threads, and the queries of one resident must run in
 *    order on the device: issue them on one stream, or order the streams. They
 *    share the resident's total and moment caches and its query-plan buffer.
 */
#ifndef QSC_H
#define QSC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qsc_status;
#define QSC_OK 0
#define QSC_ERR_INVALID_ARG -1 /* bad pointer, size, rectangle or geometry */
#define QSC_ERR_MALFORMED -2   /* a container or stream breaks FORMAT.md */
#define QSC_ERR_UNSUPPORTED -3 /* another ABI tag or format version */
#define QSC_ERR_OOM -4         /* host or device allocation failed */
#define QSC_ERR_HIP -5         /* a HIP runtime call failed */

typedef struct qsc_resident qsc_resident;
typedef struct qsc_encoder qsc_encoder;

/* Geometry of an acquisition; dtype 1 = uint8, 2 = uint16; layout 0 =
 * byte-rANS, 1 = paired tANS; scaled = 1: float32 input stored as per-block
 * calibrated uint16 codes (layout 0, dtype 2 only). */
typedef struct {
    uint32_t scan_rows, scan_cols, det_rows, det_cols;
    uint32_t dtype, layout, scaled;
} qsc_geometry;

typedef struct {
    qsc_geometry geom;
    uint32_t n_blocks;      /* ceil(scans / 512) */
    uint32_t sum_bits;      /* 32 or 64: width of masked_sum / dense_df outputs */
    uint64_t resident_bytes; /* device bytes held by the resident */
    uint64_t payload_bytes; /* encoded stream bytes */
    uint64_t mode_counts[8]; /* streams per mode number (FORMAT 2.4 / 3.4) */
    uint64_t index_bytes;   /* device bytes of the polar interaction index, 0 when none is built */
} qsc_info;

/* ABI strings of the stream layouts this library reads:
 * "qsc-byte-rans-v1;qsc-paired-v1". A container carrying another tag is
 * refused (paired-resident page, "Contract": reopen refuses another ABI). */
const char *qsc_abi(void);

/* Human-readable text of a status code. */
const char *qsc_status_string(qsc_status s);

/* ---------------------------------------------------------------- encoder
 * Host encoder (FORMAT.md), multithreaded over 512-scan blocks. Its output is
 * byte-identical to the format's reference encoder. The paired-resident page
 * ("Operation pipeline" items 1-2) has counts arrive as complete 512-scan
 * blocks and be coded per detector-pixel stream; the scaled-uint16 page has
 * float32 regions calibrated to uint16 codes before ANS coding.
 *
 * qsc_encoder_create: validates the geometry (INVALID_ARG otherwise).
 * qsc_encoder_add: host_data holds n_scans x P values, scan-major, native
 *   dtype (float32 when scaled). Scans are appended in order; every call but
 *   the last must carry a multiple of 512 scans. threads <= 0 picks the host
 *   core count. NaN/Inf in scaled input or too many scans -> INVALID_ARG.
 * qsc_encoder_size / qsc_encoder_write: once all scans are added, the blob
 *   size and a copy into caller memory of at least that many bytes.
 */
qsc_status qsc_encoder_create(const qsc_geometry *geom, qsc_encoder **out);
qsc_status qsc_encoder_add(qsc_encoder *enc, const void *host_data, uint64_t n_scans, int threads);
qsc_status qsc_encoder_size(const qsc_encoder *enc, uint64_t *nbytes);
qsc_status qsc_encoder_write(const qsc_encoder *enc, void *host_out, uint64_t capacity);
qsc_status qsc_encoder_destroy(qsc_encoder *enc);

/* ---------------------------------------------------------------- device encoder
 * The same containers, encoded on the GPU from values already in device
 * memory (paired-resident page, "Operation pipeline" items 1-2: complete
 * 512-scan blocks coded per detector-pixel stream; scaled-uint16 page: each
 * float32 region calibrated to uint16 codes first). The output is
 * byte-identical to the host encoder's, for both layouts.
 *
 * qsc_encode_device_bound: the largest container the geometry can encode to
 *   (every stream raw); a capacity that always suffices.
 * qsc_encode_device: d_data holds S x P values, scan-major, native dtype
 *   (float32 when scaled), device memory. The container is written to d_blob
 *   (device, capacity bytes) and its size to *nbytes. Temporary device memory
 *   (about 12 bytes per value, plus 2 per value when scaled) is allocated and
 *   freed inside; hip_stream is synchronised. A capacity below the size ->
 *   INVALID_ARG with *nbytes set and the payload not written; NaN or Inf in
 *   scaled input -> INVALID_ARG.
 */
qsc_status qsc_encode_device_bound(const qsc_geometry *geom, uint64_t *nbytes);
qsc_status qsc_encode_device(const qsc_geometry *geom, const void *d_data, void *d_blob, uint64_t capacity,
                             uint64_t *nbytes, void *hip_stream);

/* ---------------------------------------------------------------- resident
 * qsc_resident_create: validates a host blob (header, ABI tag, block
 *   directory, grouped offsets, table sums, every stream header: reserved
 *   bits, mode, model) and copies it to device memory on the current HIP
 *   device. host_valid (nullable) is P bytes, nonzero = valid detector pixel;
 *   NULL means every pixel is valid. Validity never changes the stored counts
 *   (quantem.widget ANS page: valid_pixels does not overwrite raw sentinels).
 *   Errors: INVALID_ARG, MALFORMED (structure), UNSUPPORTED (ABI), OOM, HIP.
 * qsc_resident_destroy: synchronises and frees everything the resident owns.
 *   The caller must destroy every resident it creates (scaled-uint16 page:
 *   the caller closes loaded residents).
 * qsc_resident_info: geometry and sizes (see qsc_info). A diagnostic helper
 *   that no passage defines: it reports the uint32/uint64 virtual-image width
 *   the paired-resident page's "Contract" fixes (row "virtual image"), the
 *   resident's device footprint (the optimization matrix page's "Memory
 *   Footprint" concern) and the per-mode stream counts.
 */
qsc_status qsc_resident_create(const void *host_blob, uint64_t nbytes, const uint8_t *host_valid,
                               void *hip_stream, qsc_resident **out);
/* qsc_resident_create_device: as qsc_resident_create for a container already
 *   in device memory (d_blob, nbytes; e.g. from qsc_encode_device). The
 *   sections before the payload (and the calibration) are copied to the host
 *   and validated there; the stream headers are validated on the device; the
 *   container is copied device to device into the resident, so d_blob may be
 *   freed afterwards. Same errors as qsc_resident_create.
 */
qsc_status qsc_resident_create_device(const void *d_blob, uint64_t nbytes, const uint8_t *host_valid,
                                      void *hip_stream, qsc_resident **out);
/* qsc_resident_create_device_borrow: as qsc_resident_create_device, but the
 *   resident uses the caller's buffer in place instead of copying it: d_blob
 *   holds the container (nbytes) within capacity bytes, and capacity must
 *   leave at least 16384 bytes after the container, which the call zeroes
 *   (the decoders read ahead into them). The caller keeps ownership and must
 *   keep the buffer alive and unchanged until the resident is destroyed. */
qsc_status qsc_resident_create_device_borrow(void *d_blob, uint64_t nbytes, uint64_t capacity,
                                             const uint8_t *host_valid, void *hip_stream, qsc_resident **out);
qsc_status qsc_resident_destroy(qsc_resident *res);
qsc_status qsc_resident_info(const qsc_resident *res, qsc_info *info);

/* ---------------------------------------------------------------- queries
 * qsc_masked_sum: virtual image out[s] = sum over p with mask[p] != 0 and
 *   valid[p] of I[s, p], exact, as uint32, or uint64 when
 *   P * maxval(dtype) > 2^32 - 1 (qsc_info.sum_bits; paired-resident page,
 *   "Contract", row "virtual image"). d_mask: device, P bytes. d_out: device,
 *   scans x (sum_bits/8) bytes. block_stride k >= 1 decodes only blocks b
 *   with b mod k == 0 (paired-resident page, "Operation pipeline" item 4);
 *   scans of the other blocks read 0.
 * qsc_dense_df: dark field out[s] = total[s] - sum over valid p with
 *   mask[p] == 0 of I[s, p], where total is the full-detector sum over valid
 *   pixels, built by a full decode on the first call and cached in the
 *   resident (optimization matrix page, "Product Coverage", row "Dense DF").
 *   Equals qsc_masked_sum with the same mask.
 * qsc_com: centre of mass in detector pixel-index units (optimization matrix
 *   page, "Product Coverage", row "CoM/DPC"): exact integer moments
 *   M0 = sum I, Mr = sum I*kr, Mc = sum I*kc over mask & valid (all valid
 *   pixels when d_mask is NULL), then row = (float)((double)Mr / M0), col
 *   likewise, 0 where M0 = 0. d_row, d_col: device float32[scans].
 * qsc_decode_region: counts of the half-open scan rectangle r0 <= r < r1,
 *   c0 <= c < c1 (scaled-uint16 page: read(scan_region=...)), written as
 *   out[((r-r0)*(c1-c0) + (c-c0)) * P + p]; invalid pixels read 0
 *   (paired-resident page, "Contract", row "diffraction pattern"). out_kind
 *   0: native dtype; 1: float32 calibrated intensity code*scale+offset of the
 *   scan's region (scaled residents only). Empty or out-of-range rectangle,
 *   or out_kind 1 on an unscaled resident -> INVALID_ARG.
 * qsc_decode_blocks: every scan of blocks first_block .. first_block +
 *   n_blocks - 1 decoded back to frames, the reconstruction feed of the
 *   paired-resident page ("Operation pipeline" item 6, decode_blocks; the
 *   feed table gives native counts and counts with a float32 square-root
 *   amplitude): out[(s - 512*first_block) * P + p]; invalid pixels read 0.
 *   out_kind 0: native dtype; 1: float32 calibrated intensity (scaled
 *   residents only); 2: float32 sqrt(count), correctly rounded. A range past
 *   the last block or a bad kind -> INVALID_ARG.
 * qsc_sum_dp: sum and mean diffraction pattern over the selected scans, the
 *   dual of a virtual image (scaled-uint16 page, "MPS implementation": mean
 *   diffraction queries accumulated straight from the encoded resident; the
 *   optimization matrix page, "Current Measured Checkpoints", gates the mean
 *   diffraction pattern as bit-exact). Selected scans: d_scan_mask[s] != 0
 *   (every scan when NULL; device, scans bytes) in the blocks block_stride
 *   visits; n is their number. d_sum[p] = exact sum of I[s, p] over them for
 *   valid p, 0 for invalid p (device uint64[P]). d_mean (nullable, device
 *   float32[P]) = (float)((double)sum / n), 0 when n = 0; for a scaled
 *   resident it is the mean of the calibrated intensities code*scale+offset,
 *   accumulated region by region in increasing order as
 *   scale_b * C_b + n_b * offset_b in float64, then divided by n and rounded
 *   to float32. The first call allocates scans/512 x P x 4 bytes of resident
 *   scratch.
 * qsc_finish: synchronises hip_stream and reports (then clears) the first
 *   malformed stream found by queries enqueued since the last check.
 * qsc_last_error: message of the resident's last failure, naming the first
 *   bad (block, pixel) for MALFORMED; valid until the next call on it. A
 *   diagnostic helper: the paired-resident page ("Contract", malformed
 *   stream) only asks that the query fail without a result; the message says
 *   which stream failed.
 */
qsc_status qsc_masked_sum(qsc_resident *res, const uint8_t *d_mask, uint32_t block_stride, void *d_out,
                          void *hip_stream, int wait);
qsc_status qsc_dense_df(qsc_resident *res, const uint8_t *d_mask, void *d_out, void *hip_stream, int wait);
qsc_status qsc_com(qsc_resident *res, const uint8_t *d_mask, float *d_row, float *d_col, void *hip_stream,
                   int wait);
/* qsc_com_noalloc: qsc_com for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc). Same arguments and results as qsc_com, but its moment
 *   partials live in a static device buffer of 3 x 1,048,576 uint64 (24 MiB)
 *   that each GPU holds until the process ends, so the call allocates
 *   nothing. A resident of more than 1,048,576 scans -> INVALID_ARG. Every
 *   call on one GPU shares that buffer: calls that overlap on a GPU (other
 *   streams, other host threads) race and must be ordered by the caller. The
 *   buffer keeps the last call's contents; each call clears the part it uses
 *   first. */
qsc_status qsc_com_noalloc(qsc_resident *res, const uint8_t *d_mask, float *d_row, float *d_col, void *hip_stream,
                           int wait);
qsc_status qsc_decode_region(qsc_resident *res, uint32_t r0, uint32_t r1, uint32_t c0, uint32_t c1, int out_kind,
                             void *d_out, void *hip_stream, int wait);
qsc_status qsc_decode_blocks(qsc_resident *res, uint32_t first_block, uint32_t n_blocks, int out_kind, void *d_out,
                             void *hip_stream, int wait);
qsc_status qsc_sum_dp(qsc_resident *res, const uint8_t *d_scan_mask, uint32_t block_stride, uint64_t *d_sum,
                      float *d_mean, void *hip_stream, int wait);
qsc_status qsc_finish(qsc_resident *res, void *hip_stream);
const char *qsc_last_error(const qsc_resident *res);

/* ---------------------------------------------------------------- block feed
 * The reconstruction feed of the paired-resident page ("Operation pipeline"
 * item 6: PairedFeed decodes whole blocks to frames for the consumer, depth
 * buffers ahead, with events both ways): blocks first_block ..
 * first_block + n_blocks - 1, blocks_per_item at a time, each item decoded as
 * by qsc_decode_blocks (out_kind, layout and invalid pixels likewise) into
 * one of the caller's depth device buffers d_bufs[0 .. depth-1] (each at
 * least blocks_per_item x 512 x P x element bytes: dtype bytes for native,
 * 4 for the float kinds) on a stream the feed creates (default priority).
 * The caller owns the buffers and must keep them until qsc_feed_destroy.
 *
 * qsc_feed_create: validates (range, item size, 1 <= depth <= 64, kind,
 *   buffers -> INVALID_ARG), orders the feed after the work already queued on
 *   consumer_stream, and queues the first depth items.
 * qsc_feed_next: the next item: consumer_stream waits for its decode (no
 *   host wait); *buf_index is its buffer, *first_scan its first scan and
 *   *n_scans its scan count, 0 after the last item. The item is the
 *   consumer's until qsc_feed_release; calling next again first ->
 *   INVALID_ARG.
 * qsc_feed_release: the consumer is done with the item as of the work queued
 *   on consumer_stream so far; its buffer then takes the item depth ahead.
 * qsc_feed_destroy: waits for the feed's decodes and frees its stream and
 *   events; MALFORMED if a decoded stream was malformed (those items' buffers
 *   hold no result). The feed's decodes use only the resident's error word
 *   and read-only tables, so queries on consumer_stream may run meanwhile.
 */
typedef struct qsc_feed qsc_feed;
qsc_status qsc_feed_create(qsc_resident *res, uint32_t first_block, uint32_t n_blocks, uint32_t blocks_per_item,
                           int out_kind, uint32_t depth, void *const *d_bufs, uint64_t buf_bytes,
                           void *consumer_stream, qsc_feed **out);
qsc_status qsc_feed_next(qsc_feed *feed, uint32_t *buf_index, uint64_t *first_scan, uint32_t *n_scans);
qsc_status qsc_feed_release(qsc_feed *feed);
qsc_status qsc_feed_destroy(qsc_feed *feed);

/* ---------------------------------------------------------------- polar interaction index
 * qsc_index_build: builds the resident's interaction index (paired-resident
 *   page, "Operation pipeline" items 3-4): the valid pixels ordered by squared
 *   distance from (center_row, center_col), then by angle atan2(dr, dc), are
 *   cut into 64-pixel leaves, and 16 consecutive leaves form a root; the exact
 *   per-scan sum of every leaf and root is bit-packed per block (each field's
 *   512 values at the width of its largest). One full decode builds it;
 *   hip_stream is synchronised. From then on qsc_masked_sum answers a mask as
 *   the index fields it covers (every valid pixel of a leaf or root selected)
 *   plus a decode of the residual pixels; results are unchanged, bit for bit.
 *   Detectors above 65,535 pixels -> UNSUPPORTED; a center outside the
 *   detector -> INVALID_ARG; a malformed stream -> MALFORMED and no index.
 *   Building again replaces the index.
 */
qsc_status qsc_index_build(qsc_resident *res, int32_t center_row, int32_t center_col, void *hip_stream);

/* qsc_masked_sum_delta: the virtual image of mask computed from that of a
 *   previous mask (paired-resident page, "Operation pipeline" item 4: a mask
 *   is decomposed as its difference from the previous mask; the baseline is
 *   kept per stride): out = prev_out + sum over mask & ~prev_mask -
 *   sum over prev_mask & ~mask, both over valid pixels of the visited blocks,
 *   exact (modular arithmetic of the output width cannot overflow the true
 *   result). d_prev_out must hold masked_sum(prev_mask, block_stride) of this
 *   resident; d_out may be d_prev_out (in place). Device pointers as in
 *   qsc_masked_sum; the first call allocates 2 x P bytes of scratch. After a
 *   failed query (MALFORMED) the caller's baseline is invalid and must be
 *   recomputed with qsc_masked_sum.
 */
qsc_status qsc_masked_sum_delta(qsc_resident *res, const uint8_t *d_prev_mask, const void *d_prev_out,
                                const uint8_t *d_mask, uint32_t block_stride, void *d_out, void *hip_stream,
                                int wait);

/* Exact encoded bytes and logical counts a masked_sum with this host mask
 * (P bytes) and stride touches: stream bytes of every selected (block, pixel)
 * plus its offset entries, and n_visited_scans x n_selected counts. This is
 * the numerator of the encoded-byte GB/s a query sustains. A measurement
 * helper that no passage defines; host-only (it reads the resident's host
 * copy of the offsets and one device copy of the validity mask). */
qsc_status qsc_query_bytes(const qsc_resident *res, const uint8_t *host_mask, uint32_t block_stride,
                           uint64_t *bytes, uint64_t *counts);

#ifdef __cplusplus
}
#endif
#endif
