// Device half of the StagQ library for gfx950 (MI355X): the decode-fused
// batch-one GEMV, the code-dump kernel, and their host dispatch.
//
// GEMV design (one launch per call):
//  * A workgroup owns a block of 16 rows (whole rows, so no atomics and no
//    second pass).  A wave step covers 16 rows x 4 consecutive tile columns:
//    lane = (tile column within the four) * 16 + row.  The S waves of the
//    workgroup split the row's groups of four tile columns between them.
//  * The 64 tiles of a wave step are one contiguous unit of the image (group
//    metadata, base chunks 0-1, planes 3..N): per step a wave reads the first
//    m + 1024 M bytes of its unit (one dwordx4 load per 1 KB chunk stretch and
//    one load of its metadata), D steps ahead of use: step 0 before the wave
//    stages its x, steps 1..D-1 right after (so across the chip every wave's
//    first step is requested before anyone's second).  All global loads go
//    through buffer resources: out-of-range offsets read zeros instead of
//    faulting.
//  * Each wave stages the x of its own tile columns in LDS (68 dwords per
//    tile: 64 of x, so the four tile columns of a step fall in different
//    banks, then the tile's sum(x) per group); a step reads its tile's x one
//    32-column quarter ahead of use.
//  * Decode: the codes of two weights are isolated into the low mantissa bits
//    of the two fp16 halves of a register (fp16 subnormals, value u * 2^-24,
//    exact), so one v_dot2_f32_f16 multiplies two codes by the natural x pair
//    (x[2i], x[2i+1]) and accumulates in fp32.  For M >= 3 the planes are first
//    merged with the base codes into 4-bit codes (Eq. 8) with shifts and
//    bit-field inserts.
//  * Per group: s_M * sum(u x) + lo_M * sum(x) (the affine collapse of Eq. 10
//    summed over the group), in fp32; the pair (lo, s) is stored per group or,
//    with codebook metadata, looked up by the group's index byte in an LDS
//    copy of the matrix's 256 pairs.
//  * Optionally x is multiplied by a per-channel inverse AWQ scale as it is
//    staged.
//  * Side record (Eq. 4): each entry carries a = P - lo - s (q - 1/2) and s, so
//    its contribution (P - W_main) x_c = (a - s 2^(1-M)) x_c needs only x_c
//    (the main stream decodes W_main = lo + s (q - 1/2 + 2^(1-M)) there because
//    its planes are zero).  The block's entries (contiguous in CSR order) are
//    spread over the lanes whatever their row and summed per row with a
//    segmented scan, so rows with many held-out weights cost no more than the
//    rest: on an extra wave of the workgroup while the others stream, or (a
//    heavy record on a small grid at 2 bits) by all waves after the main loop.
//    With fixed per-row slots instead of CSR, every slot's address is known at
//    once: a lane sums its row's slots, and no row_ptr is read.
//  * Issue order: all kernel arguments arrive in one batch of scalar loads, and
//    wave priorities favour the side-record wave, then waves in their prologue,
//    then waves in their first steps, so the waves behind catch up.
//  * Optionally the row sums are stored rounded to fp16.
//  * Row sums: the 4 S lane partials of a row, then its corrections, are added
//    in a fixed order (no atomics), so y is bitwise reproducible for a given
//    shape and M.
// A streaming-read kernel (the ceiling the GEMV is measured against) sits
// beside them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "stagq_internal.h"

namespace stagq {
namespace dev {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x80000000u;  // offset past every stream (< 2 GiB each)
// Cache policy of loads of data read once per call (the weight stream, its
// metadata and the side record): the non-temporal bit (nt) of gfx940-class
// buffer loads.  Measured on 14336 x 4096: 0.1 / 0.45 / 0.45 us faster at
// 2 / 3 / 4 bits, and a plain read of the same 17-32 MB 0.4 us faster.  x,
// which every workgroup reads, keeps the default policy.
constexpr int kStream = 2;
constexpr uint32_t kOneOne = 0x3C003C00u;  // fp16 pair (1.0, 1.0)

__device__ __forceinline__ rsrc_t mk(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 ld128s(rsrc_t r, uint32_t off) {   // streamed (read once)
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream);
}
__device__ __forceinline__ u32x2 ld64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStream);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld32s(rsrc_t r, uint32_t off) {  // streamed (read once)
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStream);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}
// dot2 into a zero accumulator: one VOP3P instruction with an inline 0, not a
// move of 0 followed by the accumulating form.
__device__ __forceinline__ float dot2z(uint32_t a, uint32_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (a & m) | (b & ~m);
}
// Pin a word as computed (one register, one bit-field insert): without it the
// compiler distributes the masks applied later into the inserts that built
// the word, which costs more instructions than the insert it saves.
__device__ __forceinline__ void keep(uint32_t& v) { asm("" : "+v"(v)); }
// Two fp16 products, each rounded once to fp16 (nearest even).
__device__ __forceinline__ uint32_t hmul2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b));
}
__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// y_r as fp32, or rounded once to fp16 (nearest even; beyond the fp16 range,
// +-inf) when the caller asked for an fp16 result.
__device__ __forceinline__ void store_y(float* y, uint16_t* y16, int r, float v) {
  if (y16) y16[r] = __builtin_bit_cast(uint16_t, (_Float16)v);
  else y[r] = v;
}
__device__ __forceinline__ uint64_t ld64side(rsrc_t r, uint32_t off) {
  const u32x2 v = ld64(r, off);
  return uint64_t(v[0]) | (uint64_t(v[1]) << 32);
}

// 2-bit fields (hi plane bit, lo plane bit) aligned with the base-stream
// dwords 2d / 2d+1 from two plane dwords d (bit 2j + e is field j of S0 dword
// 2d + e).
__device__ __forceinline__ void pair_fields(uint32_t phi, uint32_t plo, uint32_t& ev, uint32_t& od) {
  ev = bfi(0x55555555u, plo, phi << 1);
  od = bfi(0xAAAAAAAAu, phi, plo >> 1);
  keep(ev); keep(od);
}
// 4-bit codes from a high 2-bit field word and a low 2-bit field word:
// nibble m of zlo / zhi is the code of field 2m / 2m+1.
__device__ __forceinline__ void nibbles(uint32_t hw, uint32_t lw, uint32_t& zlo, uint32_t& zhi) {
  zlo = bfi(0x33333333u, lw, hw << 2);
  zhi = bfi(0xCCCCCCCCu, hw, lw >> 2);
  keep(zlo); keep(zhi);
}

struct GemvParams {
  const uint8_t* units;    // the unit array: per (block, quad) group metadata, base chunks 0-1, planes 3..N
  const uint32_t* table;   // codebook metadata: the 256 (lo | s << 16) pairs
  const uint8_t* row_ptr;
  const uint8_t* side;     // side record, one u64 per entry
  const uint32_t* x;       // fp16 pairs
  const uint32_t* xsc;     // fp16 pairs: inverse AWQ scale per input channel (scaled GEMV only)
  float* y;
  uint16_t* y16;           // fp16 result instead of y (fp16-output GEMV only)
  uint32_t unit_bytes, units_bytes, side_bytes, rp_bytes, x_bytes;
  uint32_t unit_meta;      // bytes of group metadata at the start of a unit
  int32_t R, C, T, T4, S;  // rows, cols, tiles per row (padded to a multiple of 4), waves per workgroup
  int32_t g;
  uint32_t lds_part;          // LDS offset of the lane partials (x and sum(x) at 0)
  uint32_t lds_rp, lds_runs;  // LDS offsets of the block's row_ptr and the side-record run sums
  uint32_t lds_flag;          // LDS offset of the per-wave x-staged flags (side-record wave mode)
  uint32_t lds_table;         // LDS offset of the per-wave copies of the 256 pairs (codebook metadata)
  int32_t flag_spins;         // spin limit of the side-record wave's wait for them
  int32_t slots;              // fixed side-record slots per row (0: CSR)
};

template <int M, int GU>
struct Slot {
  u32x4 a, b;                        // base stream: dwords 0..3, 4..7
  u32x4 pl[M > 2 ? M - 2 : 1];       // planes 3..M, dwords 0..3
  uint32_t meta[GU];                 // (lo | s << 16) of the tile's groups
};

// Loads of one wave step: its unit starts at byte uo (scalar) of rU; the
// lane's slot is its lane index, at voffset vW = m + 16 lane in each 1 KB
// chunk stretch (base chunk 0 at +0, chunk 1 at +1024, plane k at
// +(k - 1) 1024, scalar offsets; m the unit's metadata bytes) and vM among
// the group metadata (4 GU lane for pairs, GU lane for codebook indices, CB).
// So the step reads one contiguous piece of m + 1024 M bytes.  A step past
// the wave's last (ok false, wave-uniform) reads zeros: its voffsets are out
// of range.
template <int M, int GU, bool CB>
__device__ __forceinline__ void issue(Slot<M, GU>& s, const rsrc_t& rU, uint32_t uo, uint32_t vW,
                                      uint32_t vM, bool ok) {
  const uint32_t off = ok ? vW : kOOB;
  const int so = int(uo);
  const uint32_t offm = ok ? vM : kOOB;
  if constexpr (CB) {                    // GU index bytes, kept packed in meta[0]
    if constexpr (GU == 1)
      s.meta[0] = __builtin_amdgcn_raw_buffer_load_b8(rU, offm, so, kStream);
    else if constexpr (GU == 2)
      s.meta[0] = __builtin_amdgcn_raw_buffer_load_b16(rU, offm, so, kStream);
    else
      s.meta[0] = __builtin_amdgcn_raw_buffer_load_b32(rU, offm, so, kStream);
  } else if constexpr (GU == 1) {
    s.meta[0] = __builtin_amdgcn_raw_buffer_load_b32(rU, offm, so, kStream);
  } else if constexpr (GU == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rU, offm, so, kStream);
    s.meta[0] = v[0]; s.meta[1] = v[1];
  } else {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rU, offm, so, kStream);
    s.meta[0] = v[0]; s.meta[1] = v[1]; s.meta[2] = v[2]; s.meta[3] = v[3];
  }
  s.a = __builtin_amdgcn_raw_buffer_load_b128(rU, off, so, kStream);
  s.b = __builtin_amdgcn_raw_buffer_load_b128(rU, off, so + 1024, kStream);
#pragma unroll
  for (int k = 0; k < M - 2; k++)
    s.pl[k] = __builtin_amdgcn_raw_buffer_load_b128(rU, off, so + (k + 2) * 1024, kStream);
}

// An empty statement that reads every register of a slot: the wave waits here
// until all of the slot's loads have arrived (and nothing is computed).
template <int M, int GU>
__device__ __forceinline__ void touch(const Slot<M, GU>& s) {
  asm volatile("" :: "v"(s.a), "v"(s.b));
#pragma unroll
  for (int g = 0; g < GU; g++) asm volatile("" :: "v"(s.meta[g]));
#pragma unroll
  for (int k = 0; k < M - 2; k++) asm volatile("" :: "v"(s.pl[k]));
}

__device__ __forceinline__ uint32_t s0_dword(const u32x4& a, const u32x4& b, int dw) {
  return dw < 4 ? a[dw] : b[dw - 4];
}

// Products of one 32-column quarter d of a tile (S0 dwords 2d, 2d+1, plane
// dwords d) with its x pairs xq[0..15]; accumulators of the quarter, which
// start from zero when FIRST (the quarter opens a group).
template <int M, int GU, bool FIRST>
__device__ __forceinline__ void quarter(const Slot<M, GU>& s, int d, const uint32_t* xq,
                                        float* acc) {
  bool fresh[5] = {FIRST, FIRST, FIRST, FIRST, FIRST};
  auto mac = [&](int i, uint32_t c, uint32_t xx) {
    if (fresh[i]) {
      acc[i] = dot2z(c, xx);
      fresh[i] = false;
    } else {
      acc[i] = dot2(c, xx, acc[i]);
    }
  };
  if constexpr (M == 2) {
    // fields j = 0..4 in place (value q 2^(2j) 2^-24), 5..7 after a shift by 6.
    // A dword's eight masks issue before its eight products: alternating the
    // two costs about 10% more issue cycles per wave step (measured with two
    // waves per SIMD), 0.06 us per launch on 14336 x 4096.
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const uint32_t w = s0_dword(s.a, s.b, 2 * d + e);
      const uint32_t* x8 = xq + 8 * e;
      const uint32_t t = w >> 6;
      const uint32_t m[8] = {w & 0x00030003u, w & 0x000C000Cu, w & 0x00300030u, w & 0x00C000C0u,
                             w & 0x03000300u, t & 0x00300030u, t & 0x00C000C0u, t & 0x03000300u};
      __builtin_amdgcn_sched_barrier(0);
      mac(0, m[0], x8[0]);
      mac(1, m[1], x8[1]);
      mac(2, m[2], x8[2]);
      mac(3, m[3], x8[3]);
      mac(4, m[4], x8[4]);
      mac(2, m[5], x8[5]);
      mac(3, m[6], x8[6]);
      mac(4, m[7], x8[7]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    uint32_t ye, yo;
    const uint32_t p3 = s.pl[0][d];
    if constexpr (M >= 4) {
      pair_fields(p3, s.pl[1][d], ye, yo);
    } else {
      ye = (p3 << 1) & 0xAAAAAAAAu;
      yo = p3 & 0xAAAAAAAAu;
      keep(ye); keep(yo);
    }
    uint32_t ve = 0, vo = 0, we = 0, wo = 0;
    if constexpr (M >= 5) {
      const uint32_t p5 = s.pl[2][d];
      if constexpr (M >= 6) {
        pair_fields(p5, s.pl[3][d], ve, vo);
      } else {
        ve = (p5 << 1) & 0xAAAAAAAAu;
        vo = p5 & 0xAAAAAAAAu;
        keep(ve); keep(vo);
      }
      if constexpr (M >= 7) {
        const uint32_t p7 = s.pl[4][d];
        if constexpr (M >= 8) {
          pair_fields(p7, s.pl[5][d], we, wo);
        } else {
          we = (p7 << 1) & 0xAAAAAAAAu;
          wo = p7 & 0xAAAAAAAAu;
          keep(we); keep(wo);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 2; e++) {
      // S0 dword w = 2d + e: nibble m of z[h] (low / high half) is the code of
      // field 2m + h / 8 + 2m + h, i.e. of x pair 8w + 2m + h.
      const uint32_t* xw = xq + 8 * e;
      uint32_t z[2];
      nibbles(s0_dword(s.a, s.b, 2 * d + e), e ? yo : ye, z[0], z[1]);
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const uint32_t zz = z[h], t = zz >> 8;
        mac(0, zz & 0x000F000Fu, xw[h]);
        mac(1, zz & 0x00F000F0u, xw[2 + h]);
        mac(0, t & 0x000F000Fu, xw[4 + h]);
        mac(1, t & 0x00F000F0u, xw[6 + h]);
      }
      if constexpr (M >= 5) {
        uint32_t v[2];
        nibbles(e ? vo : ve, e ? wo : we, v[0], v[1]);
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const uint32_t zz = v[h], t = zz >> 8;
          mac(1, zz & 0x000F000Fu, xw[h]);
          mac(2, zz & 0x00F000F0u, xw[2 + h]);
          mac(1, t & 0x000F000Fu, xw[4 + h]);
          mac(2, t & 0x00F000F0u, xw[6 + h]);
        }
      }
    }
  }
}

// sum over one tile of (s_M u_M + lo_M) x, i.e. Eq. 10 summed per group.
// xl: the tile's 64 x pairs in LDS, read one quarter ahead of use, followed
// by the tile's per-group sum(x) (xl[64 + gi]).
template <int M, int GU, bool CB>
__device__ __forceinline__ float tile_partial(const Slot<M, GU>& s, const uint32_t* xl, float part,
                                              const uint32_t* tab) {
  constexpr float kM = float((1 << (M - 2)) - 1) / float(1 << (M - 1));  // (2^(M-2)-1)/2^(M-1)
  constexpr int kAcc = M == 2 ? 5 : (M >= 5 ? 3 : 2);
  float acc[GU][kAcc];
  const u32x4* xl4 = reinterpret_cast<const u32x4*>(xl);
  uint32_t xq[2][16];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const u32x4 v = xl4[k];
    xq[0][4 * k] = v[0]; xq[0][4 * k + 1] = v[1]; xq[0][4 * k + 2] = v[2]; xq[0][4 * k + 3] = v[3];
  }
#pragma unroll
  for (int d = 0; d < 4; d++) {
    if (d < 3) {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const u32x4 v = xl4[4 * (d + 1) + k];
        uint32_t* o = xq[(d + 1) & 1];
        o[4 * k] = v[0]; o[4 * k + 1] = v[1]; o[4 * k + 2] = v[2]; o[4 * k + 3] = v[3];
      }
    }
    float* a = acc[d * GU / 4];
    if (d % (4 / GU) == 0)
      quarter<M, GU, true>(s, d, xq[d & 1], a);
    else
      quarter<M, GU, false>(s, d, xq[d & 1], a);
    // An empty volatile statement that takes the quarter's accumulators and
    // clobbers memory: the quarter is computed here, and the reads of quarter
    // d + 2 cannot move above it, so at most two quarters of x are live.
    if constexpr (kAcc == 5)
      asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]) :: "memory");
    else if constexpr (kAcc == 3)
      asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]) :: "memory");
    else
      asm volatile("" : "+v"(a[0]), "+v"(a[1]) :: "memory");
  }
  const float* sx = reinterpret_cast<const float*>(xl + 64);
#pragma unroll
  for (int gi = 0; gi < GU; gi++) {
    float q;
    if constexpr (M == 2)   // s_2 sum(q x): field j accumulated at scale 2^(2j-24)
      q = acc[gi][0] * 0x1p24f + acc[gi][1] * 0x1p22f + acc[gi][2] * 0x1p20f + acc[gi][3] * 0x1p18f +
          acc[gi][4] * 0x1p16f;
    else if constexpr (M >= 5)  // s_M sum(u_M x) = s * (A 2^22 + B 2^18 + C 2^14) for every M >= 3
      q = acc[gi][0] * 0x1p22f + acc[gi][1] * 0x1p18f + acc[gi][2] * 0x1p14f;
    else
      q = acc[gi][0] * 0x1p22f + acc[gi][1] * 0x1p18f;
    // the group's pair: stored, or selected by its codebook index (CB)
    const uint32_t mw = CB ? tab[(s.meta[0] >> (8 * gi)) & 0xffu] : s.meta[gi];
    const float lo = h2f(mw & 0xffffu), st = h2f(mw >> 16);
    // s (sum u_M x) + lo_M sum(x), lo_M = lo - k_M s (Eq. 10); k_2 = 0
    const float loM = M == 2 ? lo : __builtin_fmaf(-kM, st, lo);
    part = __builtin_fmaf(st, q, part);
    part = __builtin_fmaf(loM, sx[gi], part);
  }
  return part;
}

// Add the value SH lanes down inside a 16-lane DPP row (0 where there is none).
template <int SH>
__device__ __forceinline__ float row_shr_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   0x110 + SH, 0xf, 0xf, true));
}

// One step of a segmented inclusive scan inside 16-lane rows (DPP row_shr):
// add the value SH lanes down when it belongs to the same segment r.
template <int SH>
__device__ __forceinline__ float seg_step(float v, int r) {
  const int pv = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + SH, 0xf, 0xf, true);
  const int pr = __builtin_amdgcn_update_dpp(-1, r, 0x110 + SH, 0xf, 0xf, false);
  return pr == r ? v + __builtin_bit_cast(float, pv) : v;
}
// Carry across 16-lane rows: row_bcast:15 hands lane 15 of rows 0 / 2 to rows
// 1 / 3 (row mask 0xa); row_bcast:31 hands lane 31 to rows 2 and 3 (mask 0xc).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float seg_bcast(float v, int r) {
  const int pv = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xf, false);
  const int pr = __builtin_amdgcn_update_dpp(-1, r, CTRL, ROWMASK, 0xf, false);
  return pr == r ? v + __builtin_bit_cast(float, pv) : v;
}
// Segmented inclusive scan over the 64 lanes of a wave (segment ids sorted by
// lane, every lane active): afterwards the last lane of every run of equal ids
// holds the run's sum.
__device__ __forceinline__ float seg_scan64(float v, int r) {
  v = seg_step<1>(v, r);
  v = seg_step<2>(v, r);
  v = seg_step<4>(v, r);
  v = seg_step<8>(v, r);
  v = seg_bcast<0x142, 0xa>(v, r);
  v = seg_bcast<0x143, 0xc>(v, r);
  return v;
}

constexpr int kEntries = 2;      // side-record entries prefetched per thread (in-workgroup mode)
constexpr int kSideBatches = 8;  // 64-entry batches the side-record wave keeps in flight
constexpr int kXChunks = 4;      // 16-byte x chunks staged per lane: up to 4 steps per wave
constexpr int kXPitch = 68;      // LDS dwords per tile: 64 of x, then up to 4 group sums of x

// Default spin limit of the side-record wave's wait for the staged x (about
// 60 ms); past it the wave reads x from global memory instead, which is
// equally correct.  Every main wave raises its flag right after staging, so
// the wait ends long before.
constexpr int kFlagSpins = 1 << 20;

// The side-record wave's wait for every main wave's "x staged" flag: true once
// all are up, false if the spin limit ran out first (x_c then comes from global
// memory, which gives bitwise the same values).
__device__ __forceinline__ bool wait_x_staged(const GemvParams& p, int lane, const int32_t* flag_s) {
  int spins = 0;
  while (__builtin_amdgcn_ballot_w64(lane < p.S &&
                                     __hip_atomic_load(flag_s + (lane < p.S ? lane : 0), __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_WORKGROUP) != 1) != 0) {
    if (++spins > p.flag_spins) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return spins <= p.flag_spins;
}

// Side-record wave (SIDE mode): the side record of one 16-row block, run by
// the workgroup's extra wave while the others stream the main stream.
// row_ptr -> entries are two dependent loads, and this wave issues no others,
// so its waits never queue behind weight traffic; x_c is read from the x the
// main waves stage in LDS, once every main wave has raised its flag (flag_s[w]
// = 1; all flags were cleared before the workgroup's first barrier, which this
// wave passes right after issuing its first load).  The block's entries
// (contiguous in CSR order) go 64 per batch, up to kSideBatches batches in
// flight; per batch a segmented scan by row leaves each row run's sum at its
// last lane, which adds it to the row's total in LDS (batches in order: a fixed
// summation order).
template <int M, bool SC>
__device__ __forceinline__ void side_record(const GemvParams& p, int blk, int lane, int32_t* rp_s,
                                            float* rowc_s, const int32_t* flag_s, const uint32_t* xs,
                                            const rsrc_t& rRp, const rsrc_t& rSide, const rsrc_t& rX) {
  constexpr float kHalfUlp = 2.0f / float(1 << M);   // 2^(1-M)
  const uint32_t rpv = ld32s(rRp, lane <= 16 ? uint32_t(min(blk * 16 + lane, p.R)) * 4u : kOOB);
  __builtin_amdgcn_s_barrier();          // the main waves' flags are cleared
  if (lane < 16) rowc_s[lane] = 0.f;
  const int E0 = __builtin_amdgcn_readlane(int(rpv), 0), E1 = __builtin_amdgcn_readlane(int(rpv), 16);
  if (lane <= 16) rp_s[lane] = int32_t(rpv);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bool use_lds = false;
  for (int cb = E0; cb < E1; cb += 64 * kSideBatches) {
    uint64_t ent[kSideBatches];
#pragma unroll
    for (int j = 0; j < kSideBatches; j++) {
      const int e = cb + 64 * j + lane;
      ent[j] = ld64side(rSide, e < E1 ? uint32_t(e) * 8u : kOOB);
    }
    if (cb == E0) use_lds = wait_x_staged(p, lane, flag_s);   // once, for every main wave's x
    const uint16_t* xh = reinterpret_cast<const uint16_t*>(xs);
    uint32_t xc[kSideBatches];
    if (use_lds) {
#pragma unroll
      for (int j = 0; j < kSideBatches; j++) {
        const int c = cb + 64 * j + lane < E1 ? int(ent[j] >> 48) : 0;
        xc[j] = xh[(c >> 7) * (2 * kXPitch) + (c & 127)];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSideBatches; j++) {
        const int e = cb + 64 * j + lane;
        xc[j] = ld16(rX, e < E1 ? uint32_t(ent[j] >> 48) * 2u : kOOB);
      }
      if constexpr (SC) {                // the staged x is scaled: scale these the same way
        const rsrc_t rS = mk(p.xsc, p.x_bytes);
#pragma unroll
        for (int j = 0; j < kSideBatches; j++) {
          const int e = cb + 64 * j + lane;
          xc[j] = hmul2(xc[j], ld16(rS, e < E1 ? uint32_t(ent[j] >> 48) * 2u : kOOB)) & 0xffffu;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kSideBatches; j++) {
      if (cb + 64 * j >= E1) break;      // no entries left in the block (uniform)
      const int e = cb + 64 * j + lane;
      const bool ok = e < E1;
      // row of entry e within the block: the last i with row_ptr[i] <= e
      int seg = 0;
#pragma unroll
      for (int st = 8; st >= 1; st >>= 1) seg += e >= rp_s[seg + st] ? st : 0;
      seg = ok ? seg : 16;               // 16 = no entry
      const uint64_t ev = ent[j];
      const float a = __builtin_bit_cast(float, uint32_t(ev));
      const float st = h2f(uint32_t(ev >> 32) & 0xffffu);
      float v = ok ? (a - st * kHalfUlp) * h2f(xc[j]) : 0.f;
      v = seg_scan64(v, seg);
      const int nseg = __shfl_down(seg, 1);
      if ((lane == 63 || nseg != seg) && ok) rowc_s[seg] += v;
    }
  }
}

// Side-record wave with fixed slots (p.slots = W per row): lane = j0 * 16 +
// row takes slots j0, j0 + 4, ... of its row; every address is known at once
// (no row_ptr), so the wave's first loads go out with the main waves' first
// steps.  Empty slots are zero entries (a = 0, s = 0) and add 0.  Each lane
// sums its slots in order, then the four lanes of a row are added pairwise
// (j0 0+1, 2+3, then the two sums): a fixed summation order.
template <int M, bool SC>
__device__ __forceinline__ void side_slots_wave(const GemvParams& p, int blk, int lane, float* rowc_s,
                                                const int32_t* flag_s, const uint32_t* xs,
                                                const rsrc_t& rSide, const rsrc_t& rX) {
  constexpr float kHalfUlp = 2.0f / float(1 << M);   // 2^(1-M)
  const int W = p.slots, j0 = lane >> 4;
  const uint32_t e0 = uint32_t(blk) * uint32_t(W) * 16u + uint32_t(lane & 15);
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(xs);
  float acc = 0.f;
  bool use_lds = false;
  for (int cb = 0; cb < W; cb += 4 * kSideBatches) {   // W >= 1: at least once
    uint64_t ent[kSideBatches];
#pragma unroll
    for (int t = 0; t < kSideBatches; t++) {
      const int j = cb + 4 * t + j0;
      ent[t] = ld64side(rSide, j < W ? (e0 + uint32_t(j) * 16u) * 8u : kOOB);
    }
    if (cb == 0) {
      __builtin_amdgcn_s_barrier();      // the main waves' flags are cleared
      use_lds = wait_x_staged(p, lane, flag_s);
    }
    uint32_t xc[kSideBatches];
    if (use_lds) {
#pragma unroll
      for (int t = 0; t < kSideBatches; t++) {
        const int c = int(ent[t] >> 48);   // empty and out-of-range slots: column 0
        xc[t] = xh[(c >> 7) * (2 * kXPitch) + (c & 127)];
      }
    } else {
#pragma unroll
      for (int t = 0; t < kSideBatches; t++) xc[t] = ld16(rX, uint32_t(ent[t] >> 48) * 2u);
      if constexpr (SC) {
        const rsrc_t rS = mk(p.xsc, p.x_bytes);
#pragma unroll
        for (int t = 0; t < kSideBatches; t++)
          xc[t] = hmul2(xc[t], ld16(rS, uint32_t(ent[t] >> 48) * 2u)) & 0xffffu;
      }
    }
#pragma unroll
    for (int t = 0; t < kSideBatches; t++) {
      if (cb + 4 * t >= W) break;        // no slots left (uniform)
      const uint64_t ev = ent[t];
      const float a = __builtin_bit_cast(float, uint32_t(ev));
      const float st = h2f(uint32_t(ev >> 32) & 0xffffu);
      acc += cb + 4 * t + j0 < W ? (a - st * kHalfUlp) * h2f(xc[t]) : 0.f;
    }
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) rowc_s[lane] = acc;
}

// The GEMV.  SIDE selects where the side record is applied: by an extra wave
// of the workgroup (SIDE = 1, at the highest wave priority, while the others
// stream) or by all waves after the main loop (SIDE = 0, for a heavy record on
// a small grid at 2 bits, where the main waves finish before the extra wave's
// dependent loads would).  SC: x is multiplied by the per-channel inverse AWQ scale
// p.xsc as it is staged (each product rounded once to fp16).  CB: the group
// metadata is a codebook index per group; each wave keeps its own LDS copy of
// the 256 pairs (1 KB) and looks the pair up once per group.
template <int M, int GU, int D, int SIDE, bool SC, bool CB, bool E>
__global__ void __launch_bounds__(1024) gemv_kernel(const GemvParams p) {
  extern __shared__ __align__(16) uint8_t lds[];
  uint32_t* xs = reinterpret_cast<uint32_t*>(lds);            // x pairs, tile t at t * kXPitch
  float* part_s = reinterpret_cast<float*>(lds + p.lds_part); // lane partials per wave
  int32_t* rp_s = reinterpret_cast<int32_t*>(lds + p.lds_rp); // the block's row_ptr (+ spare)
  float* runs_s = reinterpret_cast<float*>(lds + p.lds_runs); // run sums / side total per row
  int32_t* flag_s = reinterpret_cast<int32_t*>(lds + p.lds_flag); // per main wave: x staged (SIDE)

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = blockIdx.x;
  const int r = blk * 16 + (lane & 15);
  const bool row_ok = r < p.R;
  // Every kernel argument the prologue needs, in one batch of scalar loads:
  // left alone, the compiler spreads them over three waits, the last just
  // before step 0 (measured: 0.15-0.25 us slower at 3-4 bits on 14336 x 4096).
  asm volatile("" :: "s"(p.units), "s"(p.x), "s"(p.row_ptr), "s"(p.side), "s"(p.unit_bytes),
               "s"(p.units_bytes), "s"(p.x_bytes), "s"(p.rp_bytes), "s"(p.side_bytes), "s"(p.unit_meta),
               "s"(p.T), "s"(p.T4), "s"(p.S), "s"(p.R), "s"(p.slots));
  const rsrc_t rX = mk(p.x, p.x_bytes);
  const rsrc_t rRp = mk(p.row_ptr, p.rp_bytes);
  const rsrc_t rSide = mk(p.side, p.side_bytes);

  if constexpr (SIDE) {
    if (w == p.S) {                      // the side-record wave
      // Wave priorities (instruction issue on the SIMD; memory is unaffected):
      // the side-record wave first, then main waves in their prologue, then
      // in their first D steps, then the rest, so waves behind catch up with
      // those ahead and the launch's last workgroups finish sooner (measured
      // on 14336 x 4096: 0.4-0.5 us faster at 2-4 bits than equal priorities).
      __builtin_amdgcn_s_setprio(3);
      if (p.slots)
        side_slots_wave<M, SC>(p, blk, lane, runs_s, flag_s, xs, rSide, rX);
      else
        side_record<M, SC>(p, blk, lane, rp_s, runs_s, flag_s, xs, rRp, rSide, rX);
      __syncthreads();
      return;
    }
  }

  __builtin_amdgcn_s_setprio(2);                  // prologue
  const int cg = lane >> 4;                       // tile column within the four
  const int Q = (p.T + 3) >> 2;                    // groups of four tile columns
  const int q0 = (w * Q) / p.S, nq = ((w + 1) * Q) / p.S - q0;
  // the wave's first unit, and the lane's voffsets in a unit
  const uint32_t uo0 = uint32_t(blk * Q + q0) * p.unit_bytes;
  const uint32_t vW = p.unit_meta + 16u * uint32_t(lane), vM = (CB ? 1u : 4u) * GU * uint32_t(lane);
  uint32_t* tab_s = reinterpret_cast<uint32_t*>(lds + p.lds_table) + 256 * w;   // this wave's pairs (CB)
  const rsrc_t rU = mk(p.units, p.units_bytes);
  auto valid = [&](int i) { return i < nq; };   // (tile columns past the row's end are zero tiles)

  // --- prologue, in arrival order: (in-workgroup mode) the block's row_ptr,
  //     the x of this wave's tile columns, step 0 of the weights; steps
  //     1..D-1 follow once the x is staged.
  uint32_t rpv = 0;
  if constexpr (!SIDE) {
    if (!p.slots) rpv = ld32s(rRp, lane <= 16 ? uint32_t(min(blk * 16 + lane, p.R)) * 4u : kOOB);
  }
  const int cbase = 4 * q0 * 16;                         // first x chunk (8 columns) of the wave
  // x chunks of the wave's quads (those past the row's end, in its zero
  // tiles, load as zeros)
  const int nch = min(4 * nq * 16, p.T4 * 16 - cbase);
  u32x4 xv[kXChunks], av[SC ? kXChunks : 1];
#pragma unroll
  for (int k = 0; k < kXChunks; k++) {
    const int c = lane + 64 * k;
    xv[k] = ld128(rX, c < nch ? uint32_t(cbase + c) * 16u : kOOB);
  }
  if constexpr (SC) {
    const rsrc_t rS = mk(p.xsc, p.x_bytes);
#pragma unroll
    for (int k = 0; k < kXChunks; k++) {
      const int c = lane + 64 * k;
      av[k] = ld128(rS, c < nch ? uint32_t(cbase + c) * 16u : kOOB);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  Slot<M, GU> sl[E ? D + 1 : D];
  u32x4 tabv;
  if constexpr (CB) tabv = ld128(mk(p.table, 1024u), 16u * uint32_t(lane));
  issue<M, GU, CB>(sl[0], rU, uo0, vW, vM, valid(0));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SIDE) {                  // this wave's x-staged flag is cleared for the side wave
    flag_s[w] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
  }

  // --- (in-workgroup mode) the thread's first side-record entries of the
  //     block: entries E0 + j * threads + thread id, applied after the loop.
  //     Waiting for row_ptr here costs nothing: it is the wave's first load and
  //     the x below is waited for right after.
  const int tid = threadIdx.x, nthr = 64 * p.S;
  int E0 = 0, E1 = 0;
  uint64_t ent[kEntries];
  // (fixed slots: thread tid takes slots tid / 16 + j * threads / 16 of row
  // tid mod 16; no row_ptr)
  const uint32_t se0 = uint32_t(blk) * uint32_t(p.slots) * 16u + uint32_t(tid & 15);
  if constexpr (!SIDE) {
    if (p.slots) {
#pragma unroll
      for (int j = 0; j < kEntries; j++) {
        const int sj = (tid >> 4) + j * (nthr >> 4);
        ent[j] = ld64side(rSide, sj < p.slots ? (se0 + uint32_t(sj) * 16u) * 8u : kOOB);
      }
    } else {
      E0 = __builtin_amdgcn_readlane(int(rpv), 0);
      E1 = __builtin_amdgcn_readlane(int(rpv), 16);
#pragma unroll
      for (int j = 0; j < kEntries; j++) {
        const int e = E0 + j * nthr + tid;
        ent[j] = ld64side(rSide, e < E1 ? uint32_t(e) * 8u : kOOB);
      }
    }
  }

  // --- this wave's x into LDS, and sum(x) per group: a chunk holds 8
  //     columns, a group 16 / GU consecutive chunks = lanes of one DPP row,
  //     summed with row_shr steps.  Spare lanes write to spare slots so no load
  //     is sunk into a branch.  Only this wave reads these before the barrier.
  constexpr int kCpg = 16 / GU;
  const int li = lane & (kCpg - 1);
  // chunk cbase + lane + 64 k is chunk lane & 15 of tile 4 (q0 + k) + lane / 16:
  // the lane's part of both LDS addresses is fixed, the tile's is wave-uniform
  const int xl = (lane >> 4) * kXPitch + (lane & 15) * 4;
  const int sxl = li == kCpg - 1 ? (lane >> 4) * kXPitch + 64 + (lane & 15) / kCpg : -1;
  const int spare = p.T4 * kXPitch;
#pragma unroll
  for (int k = 0; k < kXChunks; k++) {
    if (64 * k >= nch) break;            // the wave's x ends here (uniform)
    const bool ok = lane + 64 * k < nch;
    const int tb = __builtin_amdgcn_readfirstlane((4 * q0 + 4 * k) * kXPitch);
    const int xo = ok ? tb + xl : spare;
    if constexpr (SC) {
#pragma unroll
      for (int i = 0; i < 4; i++) xv[k][i] = hmul2(xv[k][i], av[k][i]);
    }
    *reinterpret_cast<u32x4*>(xs + xo) = xv[k];
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) v = dot2(xv[k][i], kOneOne, v);
    float u;
    // (a group of 16 chunks is a whole DPP row, whose edges read zeros: no
    // masking; smaller groups mask the lanes that would read the group below)
    u = row_shr_add<1>(v); v = kCpg == 16 || li >= 1 ? u : v;
    u = row_shr_add<2>(v); v = kCpg == 16 || li >= 2 ? u : v;
    if constexpr (kCpg >= 8) { u = row_shr_add<4>(v); v = kCpg == 16 || li >= 4 ? u : v; }
    if constexpr (kCpg >= 16) { u = row_shr_add<8>(v); v = u; }
    // sum(x) of the lane's group sits after its tile's x (the other lanes, and
    // lanes past the wave's x, write into the spare tile)
    xs[ok && sxl >= 0 ? tb + sxl : spare + 64] = __builtin_bit_cast(uint32_t, v);
  }
  if constexpr (!SIDE) rp_s[w == 0 && lane <= 16 ? lane : 17] = int32_t(rpv);
  if constexpr (CB) *reinterpret_cast<u32x4*>(tab_s + 4 * lane) = tabv;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (SIDE) {                  // x of this wave's columns is in LDS
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __hip_atomic_store(flag_s + w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // (measured: issuing all D steps before the staging is 0.2-0.4 us slower
  // on 14336 x 4096 at 2 and 3 bits: every wave's step 0 then queues behind
  // earlier waves' later steps)
#pragma unroll
  for (int i = 1; i < D; i++) {
    issue<M, GU, CB>(sl[i], rU, uo0 + uint32_t(i) * p.unit_bytes, vW, vM, valid(i));
    __builtin_amdgcn_sched_barrier(0);
  }

  __builtin_amdgcn_s_setprio(1);                  // the first D steps
  // --- main loop; the slot of step i is reloaded with step i + D (out of
  //     range -> zeros, no traffic), which keeps every wait count
  //     path-independent.
  float part = 0.f;
  // LDS x of the lane's tile at step i: tile 4 (q0 + i) + cg (zero x past
  // the row's end, where the weights are zero tiles too).
  const int xo0 = (4 * q0 + cg) * kXPitch;
  if constexpr (E) {
    // Early issue: D steps in flight and one more slot being decoded; step
    // i + D is requested as soon as step i has arrived, before step i is
    // decoded (a wave takes at most kXChunks steps, so the loop unrolls fully).
#pragma unroll
    for (int i = 0; i < kXChunks; i++) {
      if (i == D) __builtin_amdgcn_s_setprio(0);
      Slot<M, GU>& cur = sl[i % (D + 1)];
      touch(cur);
      __builtin_amdgcn_sched_barrier(0);
      issue<M, GU, CB>(sl[(i + D) % (D + 1)], rU, uo0 + uint32_t(i + D) * p.unit_bytes, vW, vM, valid(i + D));
      __builtin_amdgcn_sched_barrier(0);
      if (i < nq) part = tile_partial<M, GU, CB>(cur, xs + xo0 + 4 * kXPitch * i, part, tab_s);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // D steps in flight; the slot of step i is reloaded with step i + D once
    // step i is decoded.
    auto step = [&](Slot<M, GU>& s, int i) {
      if (i < nq) part = tile_partial<M, GU, CB>(s, xs + xo0 + 4 * kXPitch * i, part, tab_s);
      __builtin_amdgcn_sched_barrier(0);   // reuse the slot's registers: no loads hoisted above
      issue<M, GU, CB>(s, rU, uo0 + uint32_t(i + D) * p.unit_bytes, vW, vM, valid(i + D));
    };
#pragma unroll
    for (int i = 0; i < D; i++) step(sl[i], i);
    __builtin_amdgcn_s_setprio(0);                  // the remaining steps
    for (int ib = D; ib < nq; ib += D) {
#pragma unroll
      for (int i = 0; i < D; i++) step(sl[i], ib + i);
    }
  }

  part_s[w * 64 + lane] = part;
  __syncthreads();                       // partials (and x, row_ptr or side totals) complete in LDS

  // --- row sums: lane partials in (wave, tile column) order ...
  float acc = 0.f;
  const bool owner = w == 0 && lane < 16;
  if (owner) {
    for (int k = 0; k < p.S; k++)
#pragma unroll
      for (int c = 0; c < 4; c++) acc += part_s[k * 64 + c * 16 + lane];
  }
  if constexpr (SIDE) {
    // ... then the row's side-record total from the side-record wave.
    if (owner && row_ok) store_y(p.y, p.y16, r, acc + runs_s[lane]);
    return;
  }

  // --- ... then (in-workgroup mode) the side-record corrections
  //     (a - s 2^(1-M)) x_c of the block, in entry order.  A chunk of
  //     kEntries * threads entries is spread over the threads (64 consecutive
  //     entries per wave and j); a segmented scan by row leaves, at the last
  //     lane of every row run, the run's sum; the row's owner adds its runs in
  //     order.
  constexpr float kHalfUlp = 2.0f / float(1 << M);   // 2^(1-M)
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(xs);
  if (p.slots) {
    // --- ... or (fixed slots) each thread's slots in order, then the row's
    //     owner adds the 4 S slot groups of its row in order.
    const int W = p.slots, sstep = nthr >> 4;
    float v = 0.f;
    for (int cb = 0; cb < W; cb += kEntries * sstep) {
      if (cb > 0) {                      // rare: more slots than one prefetched chunk
#pragma unroll
        for (int j = 0; j < kEntries; j++) {
          const int sj = cb + (tid >> 4) + j * sstep;
          ent[j] = ld64side(rSide, sj < W ? (se0 + uint32_t(sj) * 16u) * 8u : kOOB);
        }
      }
#pragma unroll
      for (int j = 0; j < kEntries; j++) {
        const int sj = cb + (tid >> 4) + j * sstep;
        const uint64_t ev = ent[j];
        const float a = __builtin_bit_cast(float, uint32_t(ev));
        const float st = h2f(uint32_t(ev >> 32) & 0xffffu);
        const int c = int(ev >> 48);
        if (sj < W) v += (a - st * kHalfUlp) * h2f(xh[(c >> 7) * (2 * kXPitch) + (c & 127)]);
      }
    }
    runs_s[(tid >> 4) * 17 + (tid & 15)] = v;
    __syncthreads();
    if (owner) {
      for (int k = 0; k < sstep; k++) acc += runs_s[k * 17 + lane];
      if (row_ok) store_y(p.y, p.y16, r, acc);
    }
    return;
  }
  const int echunk = kEntries * nthr;
  for (int cb = E0; cb < E1; cb += echunk) {
    if (cb > E0) {                       // rare: more entries than one prefetched chunk
      __syncthreads();                   // the previous chunk's runs are consumed
#pragma unroll
      for (int j = 0; j < kEntries; j++) {
        const int e = cb + j * nthr + tid;
        ent[j] = ld64side(rSide, e < E1 ? uint32_t(e) * 8u : kOOB);
      }
    }
#pragma unroll
    for (int j = 0; j < kEntries; j++) {
      if (cb + j * nthr >= E1) break;    // no entries left in the block (uniform)
      const int e = cb + j * nthr + tid;
      const bool ok = e < E1;
      int seg = 16;                      // rows of the block 0..15; 16 = no entry
      float v = 0.f;
      if (ok) {
        seg = 0;
#pragma unroll
        for (int i = 1; i < 16; i++) seg += e >= rp_s[i] ? 1 : 0;
        const uint64_t ev = ent[j];
        const float a = __builtin_bit_cast(float, uint32_t(ev));
        const float st = h2f(uint32_t(ev >> 32) & 0xffffu);
        const int c = int(ev >> 48);
        v = (a - st * kHalfUlp) * h2f(xh[(c >> 7) * (2 * kXPitch) + (c & 127)]);
      }
      v = seg_scan64(v, seg);
      const int nseg = __shfl_down(seg, 1);
      const bool last = lane == 63 || nseg != seg;
      runs_s[(j * p.S + w) * 17 + (last ? seg : 16)] = v;
    }
    __syncthreads();
    if (owner) {
      // the row's entries in this chunk: [max(rp, cb), min(rp+1, cb + chunk))
      const int a = max(rp_s[lane], cb) - cb, b = min(rp_s[lane + 1], cb + echunk) - cb;
      for (int q = a; q < b; q = (q | 63) + 1) acc += runs_s[(q >> 6) * 17 + lane];
    }
  }
  if (owner && row_ok) store_y(p.y, p.y16, r, acc);
}

// Streaming-read ceiling: a workgroup of 256 threads reads 16 KB (4 x 16 B per
// thread, each 4 KB piece one contiguous load across the workgroup) and
// keeps the loads alive through a checksum whose rare match writes sink.
__global__ void __launch_bounds__(256) stream_read_kernel(const uint8_t* buf, uint32_t bytes,
                                                          uint32_t* sink) {
  const rsrc_t r = mk(buf, bytes);
  const uint32_t base = blockIdx.x * 16384u + threadIdx.x * 16u;
  u32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; k++) v[k] = ld128s(r, base + 4096u * k);
  uint32_t h = 0;
#pragma unroll
  for (int k = 0; k < 4; k++) h ^= v[k][0] + v[k][1] * 3u + v[k][2] * 5u + v[k][3] * 7u;
  if (h == 0x9E3779B9u) sink[0] = h;   // data-dependent, so the loads stay
}

// Streaming read of a chosen launch shape (read-ceiling sweep): grid
// workgroups of blockDim.x threads; each pass a thread issues L 16-byte loads
// (each wave instruction one contiguous 1 KB piece, the L loads of a pass
// grid * blockDim.x * 16 bytes apart) before it uses any of them, and the
// grid strides over the buffer until every byte has been read once.
template <int L>
__global__ void __launch_bounds__(1024) stream_read_shape_kernel(const uint8_t* buf, uint32_t bytes,
                                                                 uint32_t* sink) {
  const rsrc_t r = mk(buf, bytes);
  const uint32_t lanes = gridDim.x * blockDim.x;
  const uint32_t pass = lanes * 16u * L;
  uint32_t h = 0;
  // (bytes < 2^31 and a pass never exceeds about bytes, so base cannot wrap)
  for (uint32_t base = (blockIdx.x * blockDim.x + threadIdx.x) * 16u; base < bytes; base += pass) {
    u32x4 v[L];
#pragma unroll
    for (int k = 0; k < L; k++) v[k] = ld128s(r, base + uint32_t(k) * lanes * 16u);
#pragma unroll
    for (int k = 0; k < L; k++) h ^= v[k][0] + v[k][1] * 3u + v[k][2] * 5u + v[k][3] * 7u;
  }
  if (h == 0x9E3779B9u) sink[0] = h;
}

// Code dump: one thread per (padded) tile writes the 128 codes u_M (Eq. 8) of
// its tile, read field by field from the base stream and planes 3..M.
struct CodesParams {
  const uint8_t* units;
  uint8_t* codes;
  uint32_t unit_bytes, unit_meta, units_bytes;
  int32_t R, T, Q, C;
  int64_t tiles;           // units * 64
};

template <int M>
__global__ void __launch_bounds__(256) codes_kernel(const CodesParams p) {
  const int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // unit * 64 + slot
  if (u >= p.tiles) return;
  const int64_t unit = u >> 6;
  const int t = int(u & 63);
  const int64_t row = (unit / p.Q) * 16 + (t & 15);
  const int64_t tc = (unit % p.Q) * 4 + (t >> 4);
  if (row >= p.R || tc >= p.T) return;   // padding rows and zero tiles
  const rsrc_t rU = mk(p.units, p.units_bytes);
  const uint32_t off = uint32_t(unit) * p.unit_bytes + p.unit_meta + uint32_t(t) * 16u;
  const u32x4 a = ld128(rU, off), b = ld128(rU, off + 1024u);
  u32x4 pl[M > 2 ? M - 2 : 1];
#pragma unroll
  for (int k = 0; k < M - 2; k++) pl[k] = ld128(rU, off + uint32_t(k + 2) * 1024u);
  u32x4* dst = reinterpret_cast<u32x4*>(p.codes + row * p.C + tc * 128);
#pragma unroll
  for (int i = 0; i < 8; i++) {          // columns 16i .. 16i + 15 (S0 dword i)
    const uint32_t wq = s0_dword(a, b, i);
    uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
    for (int cc = 0; cc < 16; cc++) {
      const int j = (cc >> 1) + 8 * (cc & 1);            // field of column 16i + cc
      uint32_t code = (wq >> (2 * j)) & 3u;
#pragma unroll
      for (int k = 0; k < M - 2; k++) code = (code << 1) | ((pl[k][i >> 1] >> (2 * j + (i & 1))) & 1u);
      o[cc >> 2] |= code << (8 * (cc & 3));
    }
    u32x4 v;
    v[0] = o[0]; v[1] = o[1]; v[2] = o[2]; v[3] = o[3];
    dst[i] = v;
  }
}

}  // namespace dev

// ------------------------------------------------------------- dispatch ----
struct LaunchCfg {
  int S, grid, nt_max;
  bool side;                    // side record on an extra wave (SIDE mode)
  int depth;                    // steps of loads in flight per wave (1 or 2)
  bool early;                   // early issue (step i + depth requested when step i arrives)
  size_t lds;
  dev::GemvParams prm;
};

static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

static size_t device_lds_limit() {
  static int lim = 0;
  if (!lim) {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, d) != hipSuccess || lim <= 0)
      lim = 160 * 1024;       // gfx950: 160 KB of LDS per workgroup
  }
  return size_t(lim);
}

static int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

// Loads in flight per wave ("depth") and the issue mode.  A wave requests its
// first D steps before it computes; then either (plain) the slot of step i is
// reloaded with step i + D once step i is decoded, or (early issue) step i + D
// goes out as soon as step i has arrived, into a spare slot, so the request
// overlaps the decode of step i.  On this GPU requests issued together come
// back together (with every step of a wave in flight, its first step arrives
// near the end of the whole transfer, measured per wave with s_memrealtime), so
// a shallow depth that re-issues on arrival keeps the data flowing while the
// decode follows it.  Measured in one session (us at 2 / 3 / 4 bits, the
// weight stream loaded non-temporal):
//   14336 x 4096 (3.5 blocks per CU, light record): early depth 1 5.82 / 6.63 /
//     7.69; plain depth 2 5.89 / 6.78 / 7.94; plain depth 1 7.08 / 7.88 / 8.19
//   17920 x 5120 (4.4 blocks per CU): early depth 1 8.57 / 10.34 / 11.86, plain
//     depth 2 8.66 / 10.64 / 11.90; at 5 / 6 bits plain depth 1 with one wave
//     more than the fewest 15.55 / 16.82 (early 16.19 / 17.81)
//   4096 x 4096 (1 block per CU, 65 side-record entries per block): one wave
//     more than the fewest, early depth 1 4.50 / 4.63 / 4.76 (the fewest waves,
//     plain depth 2: 5.74 / 6.30 / 6.43)
//   4096 x 14336 (1 block per CU, 229 entries per block): at 3 / 4 bits early
//     depth 1 6.88 / 8.13 (plain depth 2 7.22 / 8.25); at 2 bits, the record
//     applied after the loop, plain depth 2 6.72 (early 6.97, plain 1 7.18)
//   5120 x 17920 (1.25 blocks per CU, 573 entries per block): plain depth 1 at
//     every precision 10.92 / 12.44 / 13.83 / 19.17 / 20.33 (early 11.29 /
//     12.91 / 15.95 / 20.30 / 21.01; plain depth 2 11.15 / 13.01 / 16.19)
//   128256 x 4096 (31 blocks per CU) at 2 bits: early depth 1 36.9 us against
//     about 34 with plain depth 2, which 14336 x 4096 ties (5.89 against 5.82)
// So 2 bits keeps plain depth 2 (depth 1 on a heavy record after the loop), and
// 3 and 4 bits issue early except for a heavy record on a small grid.  Early
// issue is built for 3 and 4 bits, depth 2 for up to 3 bits.
constexpr int kHeavySide = 256;   // side-record entries per block, on average, above which depth 1 is plain
constexpr int kMaxWaves = 16;   // waves per workgroup (incl. a side-record wave): __launch_bounds__(1024)

// LDS carve-up: per tile (padded tile columns, plus a spare tile) 64 dwords
// of x and its per-group sum(x) (up to 4 dwords), per-wave lane partials, the
// block's row_ptr (plus a spare slot), side-record run sums (17 per 64-entry
// batch), per-wave x-staged flags, per-wave copies of the 256 codebook pairs.
static size_t lds_layout(int C, int S, bool cb, dev::GemvParams* prm) {
  size_t o = size_t(padded_tcols(C) + 1) * dev::kXPitch * 4;
  if (prm) prm->lds_part = uint32_t(o);
  o += size_t(S) * 64 * 4;
  if (prm) prm->lds_rp = uint32_t(o);
  o += 18 * 4;
  o = (o + 15) & ~size_t(15);
  if (prm) prm->lds_runs = uint32_t(o);
  o += size_t(std::max(dev::kEntries, 4)) * S * 17 * 4;   // CSR run sums, or 4 S slot groups
  if (prm) prm->lds_flag = uint32_t(o);
  o += size_t(kMaxWaves) * 4;
  o = (o + 15) & ~size_t(15);
  if (prm) prm->lds_table = uint32_t(o);
  if (cb) o += size_t(S) * 1024;
  return o;
}

// Launch shape: one workgroup per 16-row block, S waves splitting the row's
// groups of four tile columns, and the side record on an extra wave.  Up to 4
// bits each wave takes the most steps it can (S = ceil(groups / 4): a wave
// stages the x of at most 4 steps; measured on 14336 x 4096: 7.2 / 8.2 us at
// 2 / 3 bits against 7.6 / 8.6 with two waves per SIMD; at 4 bits, with two
// steps in flight, equal), except on grids of fewer than two blocks per CU
// with a light record, which take one wave more (4096 x 4096, see the depth
// notes above); from 5 bits S is the smallest count that puts about two waves
// on every SIMD (8 per CU), one more on grids of two or more blocks per CU,
// within [ceil(groups / 4), min(15, groups)].  The side record goes to the extra wave except for a
// heavy CSR record (more than 128 entries per block on average) on a grid of
// fewer than two workgroups per CU at 2 bits: there the main waves finish
// soonest and the side wave's chain of dependent loads would set the launch's
// end, so all waves apply the record after the loop.  Fixed slots have no
// such chain.  Measured in one session (us at 2 / 3 / 4 / 5 / 6 bits, extra
// wave against after the loop): 4096 x 4096, 65 entries per block,
// 4.65 / 4.97 / 5.04 against 4.81 / 5.19 / 5.45; 5120 x 17920, 573 per block,
// 11.7 / 13.7 / 14.7 / 19.9 / 21.3 against 11.4 / 15.9 / 15.8 / 20.9 / 22.9
// (4 bits with depth 1); 4096 x 14336, 229 per block, 7.56 / 7.95 / 8.82
// against 7.46 / 8.32 / 9.69.  With the record applied after the loop, each
// wave takes at most 3 steps (4096 x 14336: 7.23 against 7.47 us with 4;
// 5120 x 17920: 11.20 against 11.43, at 2 bits).
// STAGQ_WAVES, STAGQ_SIDE, STAGQ_DEPTH and STAGQ_EARLY override the choices
// (tuning; a depth or issue mode that is not built for the precision is
// ignored); STAGQ_FLAG_SPINS sets the side-record wave's spin limit (testing
// its global-x fallback).
constexpr int kLightSide = 128;   // side-record entries per block, on average, that the extra wave takes
static bool plan_gemv(const ImageHeader& h, int bits, LaunchCfg* c) {
  const int T = h.cols / kTileCols;
  const int Q = (T + 3) / 4;
  const int nblk = h.blocks;
  if (nblk <= 0) return false;
  const int cus = device_cus();
  const bool many = nblk >= 2 * cus;
  const bool light = h.side_slots > 0 || h.nnz <= int64_t(kLightSide) * nblk;
  bool side = many || light || bits >= 3;
  const int side_env = env_int("STAGQ_SIDE", -1);
  if (side_env == 0 || side_env == 1) side = side_env == 1;
  const int smin = (Q + dev::kXChunks - 1) / dev::kXChunks;
  // The widest rows need every wave of the workgroup for the main stream: then
  // the side record is applied after the loop instead of on an extra wave.
  if (side && smin > std::min(kMaxWaves - 1, Q) && side_env != 1) side = false;
  const int smax = std::min(kMaxWaves - (side ? 1 : 0), Q);
  if (smin > smax) return false;
  const int target = 2 * 4 * cus;
  int S = (target + nblk - 1) / nblk;
  if (side && bits <= 4) S = smin + (!many && light && !h.side_slots ? 1 : 0);
  if (side && bits >= 5 && many) S = std::max(S, smin + 1);
  if (!side) S = (Q + 2) / 3;          // after the loop: at most 3 steps per wave
  S = std::max(smin, std::min(smax, S));
  c->prm.flag_spins = env_int("STAGQ_FLAG_SPINS", dev::kFlagSpins);
  const int s_env = env_int("STAGQ_WAVES", 0);
  if (s_env) S = s_env;
  if (S < smin || S > smax) return false;
  const bool heavy = !h.side_slots && h.nnz > int64_t(kHeavySide) * nblk;
  int depth = 1;
  bool early = false;
  if (!side) depth = heavy || bits >= 4 ? 1 : 2;
  else if (bits == 2) depth = 2;
  else if (bits <= 4 && (many || !heavy)) early = true;
  const int d_env = env_int("STAGQ_DEPTH", 0), e_env = env_int("STAGQ_EARLY", -1);
  if (d_env == 1 || (d_env == 2 && bits <= 3)) depth = d_env;
  if (e_env == 0 || (e_env == 1 && (bits == 3 || bits == 4))) early = e_env == 1;
  if (early) depth = 1;
  c->S = S;
  c->side = side;
  c->depth = depth;
  c->early = early;
  c->grid = nblk;
  c->nt_max = (Q + S - 1) / S;
  c->lds = lds_layout(h.cols, S, h.codebook != 0, &c->prm);
  if (c->lds > device_lds_limit()) return false;
  c->prm.R = h.rows; c->prm.C = h.cols; c->prm.T = T; c->prm.T4 = int32_t(padded_tcols(h.cols));
  c->prm.S = S; c->prm.g = h.group;
  return true;
}

template <int M, int GU, int D, bool E>
static hipError_t launch_gemv(const LaunchCfg& c, hipStream_t st) {
  const bool sc = c.prm.xsc != nullptr, cb = c.prm.table != nullptr;
  const dim3 grid(c.grid), block(64 * (c.S + (c.side ? 1 : 0)));
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, c.lds, st, c.prm); };
  if (c.side) {
    if (cb) sc ? go(dev::gemv_kernel<M, GU, D, 1, true, true, E>) : go(dev::gemv_kernel<M, GU, D, 1, false, true, E>);
    else sc ? go(dev::gemv_kernel<M, GU, D, 1, true, false, E>) : go(dev::gemv_kernel<M, GU, D, 1, false, false, E>);
  } else {
    if (cb) sc ? go(dev::gemv_kernel<M, GU, D, 0, true, true, E>) : go(dev::gemv_kernel<M, GU, D, 0, false, true, E>);
    else sc ? go(dev::gemv_kernel<M, GU, D, 0, true, false, E>) : go(dev::gemv_kernel<M, GU, D, 0, false, false, E>);
  }
  return hipGetLastError();
}

// Instantiated depths and issue modes: early issue up to 4 bits, depth 2 up
// to 3 bits, plain depth 1 everywhere (plan_gemv picks only these).
template <int M, int GU>
static hipError_t launch_gemv_d(const LaunchCfg& c, hipStream_t st) {
  if constexpr (M == 3 || M == 4) {
    if (c.early) return launch_gemv<M, GU, 1, true>(c, st);
  }
  if constexpr (M <= 3) {
    if (c.depth == 2) return launch_gemv<M, GU, 2, false>(c, st);
  }
  return launch_gemv<M, GU, 1, false>(c, st);
}

template <int M>
static hipError_t launch_gemv_m(int GU, const LaunchCfg& c, hipStream_t st) {
  switch (GU) {
    case 1: return launch_gemv_d<M, 1>(c, st);
    case 2: return launch_gemv_d<M, 2>(c, st);
    default: return launch_gemv_d<M, 4>(c, st);
  }
}

template <int M>
static hipError_t launch_codes(const dev::CodesParams& p, hipStream_t st) {
  const unsigned blocks = unsigned((p.tiles + 255) / 256);
  hipLaunchKernelGGL((dev::codes_kernel<M>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace stagq

using namespace stagq;

extern "C" {

static int make_handle(const ImageHeader& h, const void* dev, stagq_handle* out) {
  stagq_handle hd = new (std::nothrow) stagq_handle_s;
  if (!hd) return STAGQ_EINVAL;
  hd->hdr = h;
  hd->dev = static_cast<const uint8_t*>(dev);
  *out = hd;
  return STAGQ_OK;
}

int stagq_pack(const stagq_fields* f, void* dev_buf, size_t dev_bytes, void* hip_stream,
               stagq_handle* out) {
  if (!out || !dev_buf) return STAGQ_EINVAL;
  ImageHeader h;
  int st = validate_fields(f, &h);
  if (st != STAGQ_OK) return st;
  if (reinterpret_cast<uintptr_t>(dev_buf) % 256) return STAGQ_EALIGN;
  if (dev_bytes < h.total) return STAGQ_ESIZE;
  void* host = nullptr;
  if (hipHostMalloc(&host, size_t(h.total), hipHostMallocDefault) != hipSuccess) return STAGQ_EHIP;
  st = stagq_pack_host(f, host, size_t(h.total));
  if (st == STAGQ_OK) {
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (hipMemcpyAsync(dev_buf, host, size_t(h.total), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      st = STAGQ_EHIP;
  }
  (void)hipHostFree(host);
  if (st != STAGQ_OK) return st;
  return make_handle(h, dev_buf, out);
}

int stagq_rebind(stagq_handle h, void* dev_buf, size_t dev_bytes, stagq_handle* out) {
  if (!h || !dev_buf || !out) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(dev_buf) % 256) return STAGQ_EALIGN;
  if (dev_bytes < h->hdr.total) return STAGQ_ESIZE;
  return make_handle(h->hdr, dev_buf, out);
}

int stagq_query(stagq_handle h, stagq_info* out) {
  if (!h || !out) return STAGQ_EINVAL;
  memset(out, 0, sizeof(*out));
  out->rows = h->hdr.rows; out->cols = h->hdr.cols; out->group = h->hdr.group;
  out->nbits_max = h->hdr.nbits; out->nnz = h->hdr.nnz; out->image_bytes = h->hdr.total;
  out->codebook = h->hdr.codebook;
  out->side_slots = h->hdr.side_slots;
  for (int b = 2; b <= h->hdr.nbits; b++) out->bytes_read[b] = bytes_read(h->hdr, b);
  return STAGQ_OK;
}

void stagq_destroy(stagq_handle h) { delete h; }

static int gemv_call(stagq_handle h, const void* x, const void* x_scale, bool scaled, void* y, bool half,
                     int bits, void* hip_stream) {
  if (!h) return STAGQ_EINVAL;
  const ImageHeader& H = h->hdr;
  if (bits < 2 || bits > H.nbits) return STAGQ_EBITS;
  if (H.rows == 0) return STAGQ_OK;  // nothing to compute; y may be empty
  if (!x || !y || (scaled && !x_scale)) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % (half ? 2 : 4) ||
      reinterpret_cast<uintptr_t>(x_scale) % 16)
    return STAGQ_EALIGN;
  const int GU = kTileCols / H.group;
  LaunchCfg c;
  if (!plan_gemv(H, bits, &c)) return STAGQ_ESHAPE;
  const uint8_t* b = h->dev;
  c.prm.units = b + H.off_units;
  c.prm.table = H.codebook ? reinterpret_cast<const uint32_t*>(b + H.off_table) : nullptr;
  c.prm.unit_meta = uint32_t(H.unit_meta_bytes);
  c.prm.row_ptr = b + H.off_rowptr;
  c.prm.side = b + H.off_side;
  c.prm.x = static_cast<const uint32_t*>(x);
  c.prm.xsc = scaled ? static_cast<const uint32_t*>(x_scale) : nullptr;
  c.prm.y = half ? nullptr : static_cast<float*>(y);
  c.prm.y16 = half ? static_cast<uint16_t*>(y) : nullptr;
  c.prm.unit_bytes = uint32_t(H.unit_bytes);
  c.prm.units_bytes = uint32_t(uint64_t(H.blocks) * H.quads * H.unit_bytes);
  c.prm.side_bytes = uint32_t(H.side_slots ? uint64_t(H.rows_padded) * uint64_t(H.side_slots) * 8
                                            : uint64_t(H.nnz) * 8);
  c.prm.slots = H.side_slots;
  c.prm.rp_bytes = uint32_t((int64_t(H.rows) + 1) * 4);
  c.prm.x_bytes = uint32_t(H.cols * 2);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t err;
  switch (bits) {
    case 2: err = launch_gemv_m<2>(GU, c, st); break;
    case 3: err = launch_gemv_m<3>(GU, c, st); break;
    case 4: err = launch_gemv_m<4>(GU, c, st); break;
    case 5: err = launch_gemv_m<5>(GU, c, st); break;
    case 6: err = launch_gemv_m<6>(GU, c, st); break;
    case 7: err = launch_gemv_m<7>(GU, c, st); break;
    default: err = launch_gemv_m<8>(GU, c, st); break;
  }
  return err == hipSuccess ? STAGQ_OK : STAGQ_EHIP;
}

int stagq_gemv(stagq_handle h, const void* x, float* y, int bits, void* hip_stream) {
  return gemv_call(h, x, nullptr, false, y, false, bits, hip_stream);
}

int stagq_gemv_scaled(stagq_handle h, const void* x, const void* x_scale, float* y, int bits,
                      void* hip_stream) {
  return gemv_call(h, x, x_scale, true, y, false, bits, hip_stream);
}

int stagq_gemv_f16(stagq_handle h, const void* x, const void* x_scale, void* y, int bits,
                   void* hip_stream) {
  return gemv_call(h, x, x_scale, x_scale != nullptr, y, true, bits, hip_stream);
}

int stagq_plan_gemv(int32_t rows, int32_t cols, int32_t group, int32_t nbits, int64_t nnz,
                    int32_t side_slots, int bits, int32_t* out) {
  if (!out) return STAGQ_EINVAL;
  ImageHeader H;
  if (!layout(rows, cols, group, nbits, nnz, &H, false, side_slots)) return STAGQ_ESHAPE;
  if (bits < 2 || bits > nbits) return STAGQ_EBITS;
  LaunchCfg c;
  if (!plan_gemv(H, bits, &c)) return STAGQ_ESHAPE;
  out[0] = c.grid; out[1] = 64 * (c.S + (c.side ? 1 : 0)); out[2] = c.S; out[3] = c.nt_max;
  out[4] = kBlockRows; out[5] = int32_t(c.lds); out[6] = c.side ? 1 : 0; out[7] = c.depth;
  out[8] = c.early ? 1 : 0;
  return STAGQ_OK;
}

int stagq_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream) {
  if (bytes == 0) return STAGQ_OK;
  if (!buf || !sink || bytes >= (size_t(1) << 31)) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return STAGQ_EALIGN;
  const unsigned blocks = unsigned((bytes + 16383) / 16384);
  hipLaunchKernelGGL(dev::stream_read_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), static_cast<const uint8_t*>(buf),
                     uint32_t(bytes), sink);
  return hipGetLastError() == hipSuccess ? STAGQ_OK : STAGQ_EHIP;
}

int stagq_stream_read_shape(const void* buf, size_t bytes, uint32_t* sink, int threads, int loads,
                            int grid, void* hip_stream) {
  if (bytes == 0) return STAGQ_OK;
  if (!buf || !sink || bytes >= (size_t(1) << 31)) return STAGQ_EINVAL;
  if (threads < 64 || threads > 1024 || threads % 64) return STAGQ_EINVAL;
  if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16) return STAGQ_EINVAL;
  if (grid < 0) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf) % 16) return STAGQ_EALIGN;
  const size_t per_wg = size_t(threads) * 16u * size_t(loads);
  const size_t one_pass = (bytes + per_wg - 1) / per_wg;
  const unsigned blocks = unsigned(grid == 0 ? one_pass : std::min<size_t>(size_t(grid), one_pass));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), 0, static_cast<hipStream_t>(hip_stream),
                       static_cast<const uint8_t*>(buf), uint32_t(bytes), sink);
  };
  switch (loads) {
    case 1: go(dev::stream_read_shape_kernel<1>); break;
    case 2: go(dev::stream_read_shape_kernel<2>); break;
    case 4: go(dev::stream_read_shape_kernel<4>); break;
    case 8: go(dev::stream_read_shape_kernel<8>); break;
    default: go(dev::stream_read_shape_kernel<16>); break;
  }
  return hipGetLastError() == hipSuccess ? STAGQ_OK : STAGQ_EHIP;
}

int stagq_decode_codes(stagq_handle h, int bits, uint8_t* codes, void* hip_stream) {
  if (!h) return STAGQ_EINVAL;
  const ImageHeader& H = h->hdr;
  if (bits < 2 || bits > H.nbits) return STAGQ_EBITS;
  if (H.tiles == 0) return STAGQ_OK;
  if (!codes) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(codes) % 16) return STAGQ_EALIGN;
  dev::CodesParams p;
  p.units = h->dev + H.off_units;
  p.codes = codes;
  p.unit_bytes = uint32_t(H.unit_bytes);
  p.unit_meta = uint32_t(H.unit_meta_bytes);
  p.units_bytes = uint32_t(uint64_t(H.blocks) * H.quads * H.unit_bytes);
  p.R = H.rows;
  p.T = H.cols / kTileCols;
  p.Q = H.quads;
  p.C = H.cols;
  p.tiles = H.tiles;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipError_t err;
  switch (bits) {
    case 2: err = launch_codes<2>(p, st); break;
    case 3: err = launch_codes<3>(p, st); break;
    case 4: err = launch_codes<4>(p, st); break;
    case 5: err = launch_codes<5>(p, st); break;
    case 6: err = launch_codes<6>(p, st); break;
    case 7: err = launch_codes<7>(p, st); break;
    default: err = launch_codes<8>(p, st); break;
  }
  return err == hipSuccess ? STAGQ_OK : STAGQ_EHIP;
}

}  // extern "C"
