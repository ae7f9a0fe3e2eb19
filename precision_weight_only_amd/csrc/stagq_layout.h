// Packed-image layout shared by the host packer and the gfx950 kernels.
//
// The unit of storage is a "tile": 128 consecutive input columns of one row.
// Rows are taken in blocks of 16 (the last block padded with zero rows), the
// tile columns of a row are padded with zero tiles to a multiple of 4, and
// inside a block the 16 rows of one tile column sit side by side:
//
//   tile index u = (row_block * T4 + tile_col) * 16 + (row mod 16),
//   T = cols / 128,  T4 = T rounded up to a multiple of 4
//
// so four consecutive tile columns of a row block form 64 consecutive tiles:
// the 64 lanes of a wave (16 rows x 4 tile columns) read them as one
// contiguous 1 KB piece of every stream.  Every stream is split into 16-byte
// chunks stored chunk-major (all tiles' chunk 0, then chunk 1, ...):
//
//   base stream S0   2 chunks x U tiles x 16 B   (2 bits per weight)
//   plane k = 3..N   1 chunk  x U tiles x 16 B   (1 bit per weight), plane-major
//   pairs            U x (128 / g) x 4 B          (fp16 lo | fp16 s << 16 per group)
//   row_ptr          [rows + 1] int32              (side record, CSR by row)
//   side entries     one u64 per held-out weight, in (row, col) order:
//                      bits  0..31  a = P - lo - s (q - 1/2) as fp32
//                      bits 32..47  the group step s (fp16)
//                      bits 48..63  the column
//   side values      the recorded weights P (fp16), for unpacking only
//
// Plane order puts the base first and the planes in order of k, so a read at
// precision M touches S0 and planes 3..M only (the prefix property of the
// StagQ main stream, section 3.3).
//
// Bit placement inside a tile (column c = 0..127 of the tile):
//   S0 dword w = c / 16 (dwords 0..3 in chunk 0, 4..7 in chunk 1) holds the
//       base code q of column c in field j (bits [2j, 2j+2)), where the even
//       columns 16w + 2i take fields j = i and the odd columns 16w + 2i + 1 take
//       fields j = 8 + i (i = 0..7).  Fields j and j + 8 therefore sit at the
//       same place in the two 16-bit halves of the dword and hold the natural
//       column pair (16w + 2i, 16w + 2i + 1).
//   plane dword d = c / 32 holds the plane bit of the column in S0 dword 2d + e,
//       field j, at bit 2j + e, so one shift and one bit-field insert turn two
//       planes into 2-bit fields aligned with S0 dwords 2d and 2d + 1.
#pragma once
#include <stdint.h>

namespace stagq {

constexpr int kTileCols = 128;
constexpr int kChunkBytes = 16;
constexpr int kBlockRows = 16;
constexpr int kMaxCols = 32768;   // x is staged whole in LDS (64 KB)
constexpr uint32_t kImageMagic = 0x51474153u;  // "SAGQ"
constexpr uint32_t kImageVersion = 4;
constexpr int kMaxBits = 8;

struct ImageHeader {           // first 256 bytes of an image
  uint32_t magic, version;
  int32_t rows, cols, group, nbits;
  int64_t nnz;
  int64_t tiles;               // U = padded rows * T4
  int32_t rows_padded, blocks; // rows rounded up to 16, and their 16-row blocks
  uint64_t off_s0, off_planes, off_meta, off_rowptr, off_side, off_sideval, total;
  uint64_t bytes_s0_chunk;     // U * 16
  uint64_t bytes_plane;        // U * 16
  uint64_t bytes_meta;         // U * (128 / g) * 4
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

// Tile index of (row, tile column); T4 = padded_tcols(cols).
inline int64_t tile_index(int64_t row, int64_t tcol, int64_t T4) {
  return ((row / kBlockRows) * T4 + tcol) * kBlockRows + (row % kBlockRows);
}

// Fill in every size and offset of an image; returns false for an unsupported
// shape (the caller maps that to STAGQ_ESHAPE).
inline bool layout(int32_t rows, int32_t cols, int32_t group, int32_t nbits, int64_t nnz,
                   ImageHeader* h) {
  if (rows < 0 || rows > (1 << 30) || cols <= 0 || cols % kTileCols != 0 || cols > kMaxCols)
    return false;
  if (group != 32 && group != 64 && group != 128) return false;
  if (nbits < 2 || nbits > kMaxBits) return false;
  if (nnz < 0 || nnz >= (int64_t(1) << 28)) return false;  // side record below 2 GiB
  *h = ImageHeader{};
  h->magic = kImageMagic;
  h->version = kImageVersion;
  h->rows = rows; h->cols = cols; h->group = group; h->nbits = nbits; h->nnz = nnz;
  h->blocks = (rows + kBlockRows - 1) / kBlockRows;
  h->rows_padded = h->blocks * kBlockRows;
  h->tiles = int64_t(h->rows_padded) * padded_tcols(cols);
  h->bytes_s0_chunk = uint64_t(h->tiles) * kChunkBytes;
  h->bytes_plane = uint64_t(h->tiles) * kChunkBytes;
  h->bytes_meta = uint64_t(h->tiles) * (kTileCols / group) * 4;
  const uint64_t lim = uint64_t(1) << 31;
  // The base stream and the planes are N chunk streams back to back (one
  // buffer resource covers them, with offsets below 2^31).
  if (uint64_t(nbits) * h->bytes_s0_chunk >= lim || h->bytes_meta >= lim) return false;
  uint64_t o = 256;
  h->off_s0 = o;      o = align256(o + 2 * h->bytes_s0_chunk);
  h->off_planes = o;  o = align256(o + uint64_t(nbits - 2) * h->bytes_plane);  // = off_s0 + 2 chunks
  h->off_meta = o;    o = align256(o + h->bytes_meta);
  h->off_rowptr = o;  o = align256(o + uint64_t(rows + 1) * 4);
  h->off_side = o;    o = align256(o + uint64_t(nnz) * 8);
  h->off_sideval = o; o = align256(o + uint64_t(nnz) * 2);
  h->total = o;
  return true;
}

}  // namespace stagq
