// Host-side internals shared by the packer (stagq_host.cpp) and the device
// dispatch (stagq_device.hip).
#pragma once
#include <stdint.h>
#include <string.h>

#include "stagq.h"
#include "stagq_layout.h"

struct stagq_handle_s {
  stagq::ImageHeader hdr;      // host copy of the image header
  const uint8_t* dev = nullptr;  // image base in device memory (not owned)
};

namespace stagq {

// IEEE binary16 <-> binary64 helpers (exact decode, round-to-nearest-even encode).
double half_to_double(uint16_t h);
uint16_t double_to_half(double v);

// The 256 pairs (lo | s << 16) of codebook metadata, by index i * 16 + j.
void codebook_pairs(const stagq_codebook* cb, uint32_t* out);

// Validate a field set against its layout; returns STAGQ_OK or a status.
int validate_fields(const stagq_fields* f, ImageHeader* h);

// Algorithmic bytes one GEMV at precision bits moves for this image.
uint64_t bytes_read(const ImageHeader& h, int bits);

}  // namespace stagq
