// Packed-image layout shared by the host packer and the gfx950 kernels.
//
// The unit of storage is a "tile": 128 consecutive input columns of one row.
// Rows are taken in blocks of 16 (the last block padded with zero rows), the
// tile columns of a row are padded with zero tiles to a multiple of 4 (T4),
// and the four tile columns 4j..4j+3 of a block -- 64 tiles, one wave step of
// the GEMV -- form a "unit" stored contiguously (units in order of block, then
// j):
//
//   unit (block b, quad j) at off_units + (b * Q + j) * unit_bytes,  Q = T4 / 4
//   tile (row r, tile column c) is slot t = (c mod 4) * 16 + (r mod 16) of
//   unit (r / 16, c / 4)
//
// Inside a unit, in this order (the prefix property of the StagQ main stream,
// section 3.3: a read at precision M touches the first m + 1024 M bytes of
// every unit, never the deeper planes; g' = 128 / g groups per tile):
//
//   group metadata 64 slots x g' x 4 B   (fp16 lo | fp16 s << 16 per group), or
//                  64 slots x g' x 1 B   (codebook index per group; m = 64 g')
//   base, chunk 0  64 slots x 16 B       (dwords 0..3 of the 32-byte base tile)
//   base, chunk 1  64 slots x 16 B       (dwords 4..7)
//   plane k        64 slots x 16 B       for k = 3..N (1 bit per weight)
//
// so one wave step reads one contiguous piece of m + 1024 M bytes.  With
// codebook metadata the 256 (lo | s << 16) pairs the indices select sit
// before the units (1 KB).  After the units:
//
//   row_ptr        [rows + 1] int32              (side record, CSR by row)
//   side entries   one u64 per held-out weight, in (row, col) order:
//                    bits  0..31  a = P - lo - s (q - 1/2) as fp32
//                    bits 32..47  the group step s (fp16)
//                    bits 48..63  the column
//                  or, with fixed slots (side_slots = W > 0), W slots per row
//                  in order of block, slot, row of the block: entry k of row r
//                  (in column order) at ((r / 16) W + k) 16 + r mod 16, empty
//                  slots all zero (a = 0, s = 0: a correction of 0).  The GEMV
//                  then reads the slots of a block without row_ptr.
//   side values    the recorded weights P (fp16), for unpacking only
//
// Bit placement inside a tile (column c = 0..127 of the tile):
//   base dword w = c / 16 holds the base code q of column c in field j (bits
//       [2j, 2j+2)), where the even columns 16w + 2i take fields j = i and the
//       odd columns 16w + 2i + 1 take fields j = 8 + i (i = 0..7).  Fields j and
//       j + 8 therefore sit at the same place in the two 16-bit halves of the
//       dword and hold the natural column pair (16w + 2i, 16w + 2i + 1).
//   plane dword d = c / 32 holds the plane bit of the column in base dword
//       2d + e, field j, at bit 2j + e, so one shift and one bit-field insert
//       turn two planes into 2-bit fields aligned with base dwords 2d and 2d + 1.
#pragma once
#include <stdint.h>

namespace stagq {

constexpr int kTileCols = 128;
constexpr int kBlockRows = 16;
constexpr int kMaxCols = 32768;   // x is staged whole in LDS (64 KB)
constexpr uint32_t kImageMagic = 0x51474153u;  // "SAGQ"
constexpr uint32_t kImageVersion = 6;
constexpr int kMaxSlots = 4096;        // fixed side-record slots per row, at most
constexpr int kUnitTiles = 64;         // tiles per unit: 16 rows x 4 tile columns
constexpr int kChunkStride = 1024;     // bytes of one 16-byte chunk over a unit's 64 tiles
constexpr int kMaxBits = 8;

struct ImageHeader {           // first 256 bytes of an image
  uint32_t magic, version;
  int32_t rows, cols, group, nbits;
  int64_t nnz;
  int64_t tiles;               // U = padded rows * T4
  int32_t rows_padded, blocks; // rows rounded up to 16, and their 16-row blocks
  int32_t quads, codebook;     // Q = T4 / 4 units per block; 1 = codebook metadata
  uint64_t off_units, unit_bytes, unit_meta_bytes;  // unit array; bytes per unit; metadata per unit
  uint64_t off_rowptr, off_side, off_sideval, total;
  uint64_t off_table;          // codebook metadata: the 256 pairs (0 otherwise)
  int32_t side_slots, spare;   // W > 0: fixed side-record slots per row; 0: CSR
  uint64_t pad[16];
};
static_assert(sizeof(ImageHeader) == 256, "image header is 256 bytes");

inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Position of column c (0..127) of a tile: S0 dword, field, and plane bit.
inline int col_dword(int c) { return c >> 4; }
inline int col_field(int c) { return ((c & 15) >> 1) + 8 * (c & 1); }
inline int col_plane_bit(int c) { return 2 * col_field(c) + (col_dword(c) & 1); }

// Tile columns per row in the image: cols / 128 rounded up to a multiple of 4
// (four tile columns are one contiguous piece per 16-row block).
inline int64_t padded_tcols(int64_t cols) { return ((cols / kTileCols + 3) / 4) * 4; }

// Byte offset (from the image start) of the unit holding tile (row, tile
// column), and the tile's slot in it.
inline uint64_t unit_offset(const ImageHeader& h, int64_t row, int64_t tcol) {
  return h.off_units + uint64_t((row / kBlockRows) * h.quads + tcol / 4) * h.unit_bytes;
}
inline int unit_slot(int64_t row, int64_t tcol) { return int((tcol % 4) * kBlockRows + row % kBlockRows); }
// Offsets inside a unit: metadata of group gi of slot t (its pair, or its
// codebook index byte); base dword dw (0..7) of slot t; dword d (0..3) of
// plane k (3..N) of slot t.
inline uint64_t unit_pair(const ImageHeader& h, int t, int gi) {
  return uint64_t(t) * (h.unit_meta_bytes / kUnitTiles) + uint64_t(gi) * (h.codebook ? 1 : 4);
}
inline uint64_t unit_base_dword(const ImageHeader& h, int t, int dw) {
  return h.unit_meta_bytes + uint64_t(dw >> 2) * kChunkStride + uint64_t(t) * 16 + uint64_t(dw & 3) * 4;
}
inline uint64_t unit_plane_dword(const ImageHeader& h, int k, int t, int d) {
  return h.unit_meta_bytes + uint64_t(k - 1) * kChunkStride + uint64_t(t) * 16 + uint64_t(d) * 4;
}

// Entry index of slot k of row r in a fixed-slot side record of W slots per row.
inline uint64_t slot_entry(int64_t r, int64_t k, int32_t W) {
  return (uint64_t(r / kBlockRows) * uint64_t(W) + uint64_t(k)) * kBlockRows + uint64_t(r % kBlockRows);
}

// Fill in every size and offset of an image; returns false for an unsupported
// shape (the caller maps that to STAGQ_ESHAPE).
inline bool layout(int32_t rows, int32_t cols, int32_t group, int32_t nbits, int64_t nnz,
                   ImageHeader* h, bool codebook = false, int32_t side_slots = 0) {
  if (rows < 0 || rows > (1 << 30) || cols <= 0 || cols % kTileCols != 0 || cols > kMaxCols)
    return false;
  if (group != 32 && group != 64 && group != 128) return false;
  if (nbits < 2 || nbits > kMaxBits) return false;
  if (nnz < 0 || nnz >= (int64_t(1) << 28)) return false;  // side record below 2 GiB
  if (side_slots < 0 || side_slots > kMaxSlots) return false;
  *h = ImageHeader{};
  h->magic = kImageMagic;
  h->version = kImageVersion;
  h->rows = rows; h->cols = cols; h->group = group; h->nbits = nbits; h->nnz = nnz;
  h->blocks = (rows + kBlockRows - 1) / kBlockRows;
  h->rows_padded = h->blocks * kBlockRows;
  h->tiles = int64_t(h->rows_padded) * padded_tcols(cols);
  h->quads = int32_t(padded_tcols(cols) / 4);
  h->codebook = codebook ? 1 : 0;
  h->side_slots = side_slots;
  h->unit_meta_bytes = uint64_t(kUnitTiles) * (kTileCols / group) * (codebook ? 1 : 4);
  h->unit_bytes = h->unit_meta_bytes + uint64_t(nbits) * kChunkStride;
  const uint64_t units = uint64_t(h->blocks) * h->quads;
  // One buffer resource covers the units (offsets below 2^31).
  if (units * h->unit_bytes >= (uint64_t(1) << 31)) return false;
  uint64_t o = 256;
  if (codebook) { h->off_table = o; o += 1024; }
  h->off_units = o;   o = align256(o + units * h->unit_bytes);
  h->off_rowptr = o;  o = align256(o + uint64_t(rows + 1) * 4);
  // side entries: one per held-out weight, or W slots per (padded) row
  const uint64_t side_entries = side_slots ? uint64_t(h->rows_padded) * uint64_t(side_slots) : uint64_t(nnz);
  if (side_entries * 8 >= (uint64_t(1) << 31)) return false;
  h->off_side = o;    o = align256(o + side_entries * 8);
  h->off_sideval = o; o = align256(o + uint64_t(nnz) * 2);
  h->total = o;
  return true;
}

}  // namespace stagq
