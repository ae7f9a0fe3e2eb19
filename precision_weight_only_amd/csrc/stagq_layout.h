// Packed-image layout shared by the host packer and the gfx950 kernels.
//
// The unit of work is a "tile": 128 consecutive input columns of one row
// (one lane of the GEMV owns one tile).  Tiles are numbered row-major,
// u = row * (cols / 128) + tile_col, and every stream stores tiles contiguously
// in that order, split into 16-byte chunks stored chunk-major, so that the
// lanes of a wave, which own consecutive tiles, issue fully contiguous
// dwordx4 loads:
//
//   base stream S0   2 chunks x U tiles x 16 B   (2 bits per weight)
//   plane k = 3..N   1 chunk  x U tiles x 16 B   (1 bit per weight), plane-major
//   pairs            rows * (cols / g) x 4 B     (fp16 lo | fp16 s << 16)
//   side record      row_ptr [rows+1] i32, and per entry one u64:
//                    bits 0..29 col, 30..31 base code q at (row, col),
//                    32..47 the recorded weight (fp16), 48..63 row mod 2^16
//                    (a workgroup owning fewer than 2^16 consecutive rows
//                    recovers the full row from its first row)
//
// Plane order puts the base first and the planes in order of k, so a read at
// precision M touches S0 and planes 3..M only (the prefix property of the
// StagQ main stream, section 3.3).
//
// Bit placement inside a tile (columns c = 0..127 of the tile, d = c / 32):
//   S0 dword 2d + e (e = 0, 1; dwords 0..3 in chunk 0, 4..7 in chunk 1)
//       holds in bits [2j, 2j+2) the base code q of column 32d + 2j + e,
//       j = 0..15: even columns of the 32-column block in dword 2d, odd in 2d+1.
//   plane dword d holds in bit t the plane bit of column 32d + t.
// With this placement the kernel merges a plane pair into 2-bit fields aligned
// with S0 by one shift and one bit-field insert per 32 weights, and merges
// those with S0 into 4-bit codes with the same two operations per 16 weights.
#pragma once
#include <stdint.h>

namespace stagq {

constexpr int kTileCols = 128;
constexpr int kChunkBytes = 16;
constexpr uint32_t kImageMagic = 0x51474153u;  // "SAGQ"
constexpr uint32_t kImageVersion = 2;
constexpr int kMaxBits = 8;

struct ImageHeader {           // first 256 bytes of an image
  uint32_t magic, version;
  int32_t rows, cols, group, nbits;
  int64_t nnz;
  int64_t tiles;               // U = rows * cols / 128
  uint64_t off_s0, off_planes, off_meta, off_rowptr, off_side, off_unused, total;
  uint64_t bytes_s0_chunk;     // U * 16
  uint64_t bytes_plane;        // U * 16
  uint64_t bytes_meta;         // rows * cols / group * 4
  uint64_t pad[17];
};
static_assert(sizeof(ImageHeader) == 256, "image header is 256 bytes");

inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Fill in every size and offset of an image; returns false for an unsupported
// shape (the caller maps that to STAGQ_ESHAPE).
inline bool layout(int32_t rows, int32_t cols, int32_t group, int32_t nbits, int64_t nnz,
                   ImageHeader* h) {
  if (rows < 0 || cols <= 0 || cols % kTileCols != 0) return false;
  if (group != 32 && group != 64 && group != 128) return false;
  if (nbits < 2 || nbits > kMaxBits) return false;
  if (nnz < 0 || nnz >= (int64_t(1) << 28)) return false;  // side record below 2 GiB
  if (cols >= (1 << 30)) return false;
  *h = ImageHeader{};
  h->magic = kImageMagic;
  h->version = kImageVersion;
  h->rows = rows; h->cols = cols; h->group = group; h->nbits = nbits; h->nnz = nnz;
  h->tiles = int64_t(rows) * (cols / kTileCols);
  h->bytes_s0_chunk = uint64_t(h->tiles) * kChunkBytes;
  h->bytes_plane = uint64_t(h->tiles) * kChunkBytes;
  h->bytes_meta = uint64_t(rows) * (cols / group) * 4;
  const uint64_t lim = uint64_t(1) << 31;
  if (h->bytes_s0_chunk >= lim || h->bytes_meta >= lim) return false;
  uint64_t o = 256;
  h->off_s0 = o;      o = align256(o + 2 * h->bytes_s0_chunk);
  h->off_planes = o;  o = align256(o + uint64_t(nbits - 2) * h->bytes_plane);
  h->off_meta = o;    o = align256(o + h->bytes_meta);
  h->off_rowptr = o;  o = align256(o + uint64_t(rows + 1) * 4);
  h->off_side = o;    o = align256(o + uint64_t(nnz) * 8);
  h->off_unused = o;
  h->total = o;
  return true;
}

}  // namespace stagq
