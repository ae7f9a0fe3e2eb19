/*
 * stagq.h -- C ABI of the StagQ batch-one GEMV library for AMD Instinct MI355X
 * (gfx950).
 *
 * StagQ ("StagQ: Constraint-Driven Multi-Precision Weight Quantization for
 * LLMs") stores a weight matrix once as a multi-precision main stream plus a
 * sparse side record:
 *   - a 2-bit group-wise affine base code q in {0..3} (section 3.3),
 *   - 1-bit refinement planes b_k, k = 3..N, each the sign of the residual
 *     left by the preceding prefix, on the dyadic half-step schedule
 *     t_k = s / 2^(k-1) (section 3.2, Eq. 7),
 *   - one (lo, s) pair per group of g consecutive input columns, shared by
 *     every precision (section 3.1),
 *   - a side record P of held-out weights (section 3, Eq. 4).
 * A read at precision M (2 <= M <= N) decodes the composite integer
 * u_M = q 2^(M-2) + sum_{k=3..M} b_k 2^(M-k) (Eq. 8) through one affine map,
 * W_main = lo_M + s_M u_M with s_M = s / 2^(M-2) and
 * lo_M = lo - s (2^(M-2) - 1) / 2^(M-1) (section 3.4, Eq. 10), and the complete
 * reconstruction is (1 - m) * W_main + P (Eq. 4).
 *
 * Matrices are rows (output channels) x cols (input channels); a group is g
 * consecutive columns of one row.  Supported: cols a positive multiple of 128
 * up to 32768, g in {32, 64, 128}, 2 <= N <= 8, every device stream below 2 GiB.
 *
 * Conventions for every call:
 *   - Return value: STAGQ_OK (0) or a negative STAGQ_E* status.  Arguments are
 *     validated on the host before anything is launched; no C++ exception
 *     crosses this interface.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP device
 *     memory on the current device.  A hip_stream of NULL means the default
 *     stream.
 *   - fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 */
#ifndef STAGQ_H
#define STAGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STAGQ_OK       0
#define STAGQ_EINVAL  (-1)  /* null pointer, zero size where one is needed, bad argument */
#define STAGQ_EBITS   (-2)  /* bits outside [2, N] */
#define STAGQ_ESHAPE  (-3)  /* unsupported rows/cols/group/N, or a stream >= 2 GiB */
#define STAGQ_ECSR    (-4)  /* malformed side record (row_ptr, col order/range), or fixed
                               slots fewer than the fullest row's entries or above 4096 */
#define STAGQ_EALIGN  (-5)  /* pointer not aligned as documented */
#define STAGQ_EHIP    (-6)  /* a HIP runtime call failed */
#define STAGQ_EFIELD  (-7)  /* field out of range: q > 3, plane bit > 1, plane bit set at a
                               held-out position, non-finite lo or s */
#define STAGQ_ESIZE   (-8)  /* destination buffer too small / image size mismatch */
#define STAGQ_EIMAGE  (-9)  /* packed image header not recognised */

typedef struct stagq_handle_s* stagq_handle;

/*
 * Codebook metadata ([StagQ] section 3.1, Appendix G): two 16-entry fp16
 * codebooks per matrix, one of log2 s and one of lo / s, and per group an
 * 8-bit index i * 16 + j.  The pair of index i * 16 + j is
 * s = fp16(2^log2s[i]), lo = fp16(ratio[j] * s), each rounded once to nearest.
 *   idx    [rows*(cols/group)]   uint8 index per group
 *   log2s  [16], ratio [16]       fp16 bits
 * Host memory, caller-owned, read during the call only.
 */
typedef struct {
  const uint8_t* idx;
  const uint16_t* log2s;
  const uint16_t* ratio;
} stagq_codebook;

/*
 * Unpacked encoder output in host memory, caller-owned, read during the call
 * only.  Layouts are row-major.
 *   q        [rows*cols]                 base codes 0..3
 *   planes   [(N-2)*rows*cols]           refinement bits 0/1, plane k = 3 first
 *   lo, s    [rows*(cols/group)]         fp16 bits of the group pair
 *   row_ptr  [rows+1], col [nnz], val [nnz]: the side record P as CSR sorted by
 *            (row, col); val holds the fp16 bits of the recorded weight.
 *   codebook NULL: the image stores lo, s (4 bytes per group).  Otherwise the
 *            image stores the codebook metadata (1 byte per group, plus the 256
 *            pairs once), and lo, s must be the pairs the indices select.
 *   side_slots  how the image stores the side record: 0 as CSR (row_ptr and
 *            one entry per held-out weight; the GEMV reads row_ptr, then the
 *            entries); W > 0 as W fixed slots per row ([StagQ] Appendix A and
 *            Appendix E: the per-row slots the pages' kernel reads on the
 *            feed-forward matrices), W at least the fullest row's count
 *            (else STAGQ_ECSR) and at most 4096; -1 for W = the fullest row's
 *            count (0 entries: CSR).  Fixed slots cost W * 8 bytes per row
 *            whatever the row holds, and spare the GEMV the dependent row_ptr
 *            read.
 * The planes must be 0 at held-out positions (section 3.6: the planes skip every
 * position the side record carries); q there is the base code of the original
 * weight.
 */
typedef struct {
  int32_t rows, cols, group, nbits_max;
  const uint8_t* q;
  const uint8_t* planes;
  const uint16_t* lo;
  const uint16_t* s;
  const int32_t* row_ptr;
  const int32_t* col;
  const uint16_t* val;
  int64_t nnz;
  const stagq_codebook* codebook;
  int32_t side_slots;
} stagq_fields;

/* Shape and traffic of a packed matrix. */
typedef struct {
  int32_t rows, cols, group, nbits_max;
  int64_t nnz;
  uint64_t image_bytes;      /* size of the packed image */
  /* Algorithmic bytes one GEMV at precision b moves, for b = 2..N (index b;
   * 0 elsewhere): base stream + planes 3..b + group metadata (4 bytes per group,
   * or 1 byte per group plus the 1 KB table of 256 pairs) + side record (CSR:
   * row_ptr and one 8-byte entry per held-out weight; fixed slots: 8 bytes per
   * slot of every row) + x (fp16) + y (fp32). */
  uint64_t bytes_read[9];
  int32_t codebook;          /* 1 if the image stores codebook metadata */
  int32_t side_slots;        /* fixed side-record slots per row; 0 for CSR */
} stagq_info;

/* Bytes of the packed image for these fields (0 if the shape is unsupported). */
size_t stagq_packed_bytes(const stagq_fields* f);

/*
 * Validate f and write its packed image into host memory dst (dst_bytes >=
 * stagq_packed_bytes(f), 16-byte aligned).  Pure host code: no HIP call.  The
 * image is plane-major per unit of 16 rows x 4 tiles of 128 columns: the group
 * metadata, the base stream, then plane 3, 4, ..., N, so a read at precision M
 * touches only the metadata, the base and planes 3..M of every unit (section
 * 3.3: fields stored in plane order); the side record follows the units.
 */
int stagq_pack_host(const stagq_fields* f, void* dst, size_t dst_bytes);

/*
 * Validate f, build the packed image and copy it into caller-owned device
 * memory dev_buf (dev_bytes >= stagq_packed_bytes(f), 256-byte aligned), on
 * hip_stream; returns once the copy has completed (the call synchronises
 * hip_stream).  *out receives a new handle: a host-side descriptor that refers
 * to dev_buf without owning it.  dev_buf must outlive the handle.
 */
int stagq_pack(const stagq_fields* f, void* dev_buf, size_t dev_bytes, void* hip_stream,
               stagq_handle* out);

/*
 * New handle for another device buffer that already holds a byte-identical copy
 * of the image behind h (for instance several copies for cache-cold timing).
 * dev_buf is 256-byte aligned and at least the image size; not owned.
 */
int stagq_rebind(stagq_handle h, void* dev_buf, size_t dev_bytes, stagq_handle* out);

/*
 * y = W_hat^(bits) x (Eq. 4 with Eq. 10), batch one.
 *   x    device, fp16 [cols], 16-byte aligned
 *   y    device, fp32 [rows], 4-byte aligned (written, not accumulated)
 *        (with rows == 0 the call does nothing and x, y may be NULL)
 *   bits precision M of this call, 2 <= bits <= N; any call may pick any M on
 *        the same handle (one stream serves every precision).
 * One kernel launch on hip_stream; asynchronous (no synchronisation), no
 * allocation.  The result is deterministic for a given shape and bits (fixed
 * summation order, no atomics).  Handles are immutable, so calls on different
 * streams may run concurrently.
 */
int stagq_gemv(stagq_handle h, const void* x, float* y, int bits, void* hip_stream);

/*
 * The GEMV with the inverse activation-aware (AWQ) scale applied to x at run
 * time ([StagQ] section 3.6 and Appendix E: the quantizer worked on W diag(a),
 * so the decoder multiplies input channel c by 1 / a_c where no preceding
 * normalization absorbs it):  y = W_hat^(bits) x',  x'_c = fp16(x_c * x_scale_c),
 * each product rounded once to fp16 (nearest even) as x is staged.
 *   x_scale  device, fp16 [cols], 16-byte aligned: the factors 1 / a_c
 * Everything else as stagq_gemv (same launch, same cost but one more 2-byte
 * read per column); STAGQ_EINVAL for a NULL x_scale, STAGQ_EALIGN for a
 * misaligned one.
 */
int stagq_gemv_scaled(stagq_handle h, const void* x, const void* x_scale, float* y, int bits,
                      void* hip_stream);

/*
 * The GEMV with an fp16 result, for a consumer that takes fp16 activations:
 * y_r = fp16(the fp32 row sum stagq_gemv or stagq_gemv_scaled would write),
 * rounded once to nearest even in the same launch (no second pass over y);
 * a row sum of magnitude 65520 or more becomes +-inf.
 *   x_scale  NULL for no activation scale, else the inverse AWQ scale as in
 *            stagq_gemv_scaled (device fp16 [cols], 16-byte aligned)
 *   y        device, fp16 [rows], 2-byte aligned (written, not accumulated)
 * Same launch, cost and determinism as stagq_gemv, with 2 bytes written per
 * row instead of 4.  ([StagQ] Appendix G: the pages' kernel accumulates in
 * half precision and adds into a half-precision output with atomics; here the
 * sums stay fp32 in a fixed order and only the stored value is fp16.)
 */
int stagq_gemv_f16(stagq_handle h, const void* x, const void* x_scale, void* y, int bits,
                   void* hip_stream);

/*
 * Write the composite integers u_bits (Eq. 8) of the main stream, read field
 * by field from the packed image by a kernel of its own (the GEMV decodes
 * them with different arithmetic; its decode is checked through y):
 * codes is device uint8 [rows*cols], row-major, 16-byte aligned.
 * Asynchronous on hip_stream.  (Held-out positions decode like any other: q
 * followed by zero planes.)
 */
int stagq_decode_codes(stagq_handle h, int bits, uint8_t* codes, void* hip_stream);

/*
 * Launch shape the GEMV uses for a matrix of this shape, side-record size nnz
 * and side-record format (side_slots as in stagq_fields, resolved: 0 CSR, W > 0
 * fixed slots) at precision bits (on the current device, or assuming 256
 * compute units when none is present):
 * out[0] workgroups (one per 16-row block), out[1] threads per workgroup,
 * out[2] waves per workgroup that stream the main stream, out[3] steps per
 * such wave (a step is 16 rows x 4 tile columns of 128), out[4] rows per
 * workgroup, out[5] LDS bytes, out[6] 1 if the side record runs on an extra
 * wave of each workgroup (else 0), out[7] steps of loads in flight per wave,
 * out[8] 1 if a wave requests its next step as soon as the current one has
 * arrived (early issue; else once it is decoded).  out is host int32[9].
 * Pure host logic.
 */
int stagq_plan_gemv(int32_t rows, int32_t cols, int32_t group, int32_t nbits, int64_t nnz,
                    int32_t side_slots, int bits, int32_t* out);

/*
 * Streaming-read ceiling (measurement aid, not part of the method): read bytes
 * of device memory at buf once, 16-byte loads with the non-temporal cache
 * policy the GEMV uses for its weight stream, 16 KB per 256-thread
 * workgroup, and discard them (sink, device uint32 [1], is written only when
 * a checksum of the data hits one 32-bit value, which keeps the loads alive).  Timing this on
 * the byte count a GEMV moves gives the plain-read time of those bytes on this
 * GPU.  buf 16-byte aligned, bytes < 2^31; bytes == 0 does nothing.  One
 * launch on hip_stream, asynchronous.  STAGQ_EINVAL for NULL pointers or
 * bytes >= 2^31, STAGQ_EALIGN for a misaligned buf, STAGQ_EHIP on a launch
 * error.
 */
int stagq_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream);

/*
 * Streaming read of a chosen launch shape (measurement aid for the read-ceiling
 * sweep, not part of the method): grid workgroups of threads threads each
 * (a multiple of 64 in [64, 1024]); in every pass a thread issues loads
 * (1, 2, 4, 8 or 16) 16-byte non-temporal loads before it uses them, every wave instruction
 * one contiguous 1 KB piece, and the grid strides over buf until all bytes
 * have been read once.  grid == 0 launches as many workgroups as one pass
 * needs (ceil(bytes / (threads * loads * 16))); a smaller grid makes a
 * persistent read of several passes.  Data are discarded as in
 * stagq_stream_read (sink written only on one checksum value).  buf 16-byte
 * aligned, bytes < 2^31; bytes == 0 does nothing.  STAGQ_EINVAL for NULL
 * pointers, a byte count >= 2^31 or a shape outside these sets, STAGQ_EALIGN,
 * STAGQ_EHIP on a launch error.
 */
int stagq_stream_read_shape(const void* buf, size_t bytes, uint32_t* sink, int threads, int loads,
                            int grid, void* hip_stream);

/* Fill *out with shape and per-precision traffic of h. */
int stagq_query(stagq_handle h, stagq_info* out);

/* Release the host descriptor (never frees device memory).  NULL is a no-op. */
void stagq_destroy(stagq_handle h);

/* Static description of a status code. */
const char* stagq_strerror(int status);

/*
 * Reference-grade encoder of the library (host, multi-threaded), following the
 * encoder of section 3.6 / Appendix E without calibration data: ratio-criterion
 * pre-grid guard (at most one entry per group whose magnitude exceeds ratio_T
 * times the group's second largest, ranked by that ratio), min-max pair fit over
 * the remaining entries stored as fp16, nearest base code (ties upward),
 * post-grid guard, and planes that store the sign of the residual of the
 * preceding prefix (sign(0) = +1), skipping held-out positions.
 *   budget        side-record size K (post_per_row = 0), or the cap of the
 *                 pre-grid guard alone (post_per_row > 0)
 *   post_per_row  0: the post-grid guard fills the budget with the largest
 *                 two-bit residuals |w - (lo + s q)| of the matrix (ties by
 *                 flat index); k > 0: it takes the k largest of every row (ties
 *                 by column; [StagQ] Appendix E picks per output row, there
 *                 activation-weighted; here every channel weighs the same)
 *   w       host fp16 [rows*cols]
 *   outputs host, caller-allocated: q [rows*cols], planes [(N-2)*rows*cols],
 *           lo, s [rows*cols/group], row_ptr [rows+1], col and val
 *           [budget + rows*post_per_row] (row_ptr[rows] entries are written);
 *           *n_pre receives how many entries the pre-grid guard took.
 * group may be any divisor of cols here (packing restricts it further).
 */
int stagq_encode(const uint16_t* w, int32_t rows, int32_t cols, int32_t group, int32_t nbits,
                 int64_t budget, double ratio_T, int32_t post_per_row, uint8_t* q, uint8_t* planes,
                 uint16_t* lo, uint16_t* s, int32_t* row_ptr, int32_t* col, uint16_t* val,
                 int64_t* n_pre);

/*
 * Inverse of stagq_pack_host for a host copy of an image (layout round-trip
 * checks): writes the fields into caller-allocated host arrays sized as in
 * stagq_fields (the shape is read from the image header into *shape).
 */
int stagq_unpack_host(const void* image, size_t image_bytes, stagq_info* shape, uint8_t* q,
                      uint8_t* planes, uint16_t* lo, uint16_t* s, int32_t* row_ptr, int32_t* col,
                      uint16_t* val);

#ifdef __cplusplus
}
#endif

#endif /* STAGQ_H */
