// Device half of the StagQ library for gfx950 (MI355X): the decode-fused
// batch-one GEMV, the code-dump kernel, and their host dispatch.
//
// GEMV design (one launch per call):
//  * A lane owns one 128-column tile of one row.  A workgroup of k waves runs
//    `rpp` rows side by side (rpp * tiles_per_row <= 64k lanes) for NP passes,
//    so it owns RB = NP * rpp consecutive rows and a contiguous range of every
//    stream.  All global loads go through buffer resources: out-of-range lanes
//    read zeros instead of faulting.
//  * x (fp16) is staged once into LDS, then each lane keeps the 128 values of
//    its tile in 64 VGPRs as fp16 pairs, permuted to match the bit placement of
//    the packed stream (see stagq_layout.h).
//  * Per pass a lane fetches its tile's base stream (2 x dwordx4), planes 3..M
//    (1 x dwordx4 each) and group pairs, D passes ahead of use.
//  * Decode: the codes of two weights are isolated into the low mantissa bits
//    of the two fp16 halves of a register (fp16 subnormals, value u * 2^-24,
//    exact), so one v_dot2_f32_f16 multiplies two codes by two x values and
//    accumulates in fp32.  For M >= 3 the planes are first merged with the base
//    codes into 4-bit codes (Eq. 8) with shifts and bit-field inserts.
//  * Per tile and group: partial = s_M * sum(u x) + lo_M * sum(x) (the affine
//    collapse of Eq. 10 summed over the group), in fp32.
//  * Side record (Eq. 4): each entry contributes (P - W_main) x_c, where the
//    main stream decodes W_main = lo + s (q - 1/2 + 2^(1-M)) there because its
//    planes are zero.  Entries are prefetched in the prologue and corrected at
//    the end from LDS copies of the group pairs and x.
//  * Row sums: fixed-order sums of the tile partials and the row's corrections
//    (no atomics), so y is bitwise reproducible for a given shape and M.
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
constexpr int kXChunks = 8;             // x staging: up to 8 dwordx4 per thread
constexpr int kEntries = 4;             // side-record entries prefetched per thread
constexpr uint32_t kOneOne = 0x3C003C00u;  // fp16 pair (1.0, 1.0)

__device__ __forceinline__ rsrc_t mk(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 ld64(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
  return (a & m) | (b & ~m);
}
__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
// fp16 pair (x[a], x[b]) from raw pairs xr[i] = (x[2i], x[2i+1]).
__device__ __forceinline__ uint32_t pick(const uint32_t* xr, int a, int b) {
  const uint32_t lo = (xr[a >> 1] >> ((a & 1) * 16)) & 0xffffu;
  const uint32_t hi = (xr[b >> 1] >> ((b & 1) * 16)) & 0xffffu;
  return lo | (hi << 16);
}

// 2-bit fields (hi plane bit, lo plane bit) for the even / odd columns of a
// 32-column block, aligned with the base-stream dwords 2d / 2d+1.
__device__ __forceinline__ void pair_fields(uint32_t phi, uint32_t plo, uint32_t& ev, uint32_t& od) {
  ev = bfi(0x55555555u, plo, phi << 1);
  od = bfi(0xAAAAAAAAu, phi, plo >> 1);
}
// 4-bit codes from a high 2-bit field word and a low 2-bit field word:
// nibble m of zlo / zhi is the code of field 2m / 2m+1.
__device__ __forceinline__ void nibbles(uint32_t hw, uint32_t lw, uint32_t& zlo, uint32_t& zhi) {
  zlo = bfi(0x33333333u, lw, hw << 2);
  zhi = bfi(0xCCCCCCCCu, hw, lw >> 2);
}

struct GemvParams {
  const uint8_t* s0;       // base stream, chunk 0 (chunk 1 follows at +chunk_bytes)
  const uint8_t* planes;   // plane 3 (plane k at +(k-3)*chunk_bytes)
  const uint8_t* meta;
  const uint8_t* row_ptr;
  const uint8_t* side;     // side record, one u64 per entry
  const uint8_t* x;
  float* y;
  uint32_t chunk_bytes, meta_bytes, side_bytes, rp_bytes, x_bytes;
  int32_t R, C, T, g, rpp, P, NP, RB;
  int32_t red;             // tiles per row when rows are reduced in the loop (T | 64), else 0
  int32_t ppitch;          // LDS floats per row of tile partials (T + 1) when red == 0
  uint32_t lds_rp, lds_meta, lds_part, lds_corr;
};

template <int M, int GU>
struct Slot {
  u32x4 a, b;                        // base stream: dwords 0..3, 4..7
  u32x4 pl[M > 2 ? M - 2 : 1];       // planes 3..M, dwords 0..3
  uint32_t meta[GU];                 // (lo | s << 16) of the tile's groups
};

template <int M, int GU>
__device__ __forceinline__ void issue(Slot<M, GU>& s, const rsrc_t& rA, const rsrc_t& rB,
                                      const rsrc_t* rP, const rsrc_t& rMeta, uint32_t tile, bool ok) {
  const uint32_t off = ok ? tile * 16u : kOOB;
  s.a = ld128(rA, off);
  s.b = ld128(rB, off);
#pragma unroll
  for (int k = 0; k < M - 2; k++) s.pl[k] = ld128(rP[k], off);
  const uint32_t offm = ok ? tile * (4u * GU) : kOOB;
  if constexpr (GU == 1) {
    s.meta[0] = ld32(rMeta, offm);
  } else if constexpr (GU == 2) {
    u32x2 v = ld64(rMeta, offm);
    s.meta[0] = v[0]; s.meta[1] = v[1];
  } else {
    u32x4 v = ld128(rMeta, offm);
    s.meta[0] = v[0]; s.meta[1] = v[1]; s.meta[2] = v[2]; s.meta[3] = v[3];
  }
}

__device__ __forceinline__ uint32_t s0_dword(const u32x4& a, const u32x4& b, int dw) {
  return dw < 4 ? a[dw] : b[dw - 4];
}

// sum over the tile of (s_M u_M + lo_M) x, i.e. Eq. 10 summed per group.
template <int M, int GU>
__device__ __forceinline__ float tile_partial(const Slot<M, GU>& s, const uint32_t* xp, const float* sx) {
  constexpr float kM = float((1 << (M - 2)) - 1) / float(1 << (M - 1));  // (2^(M-2)-1)/2^(M-1)
  float sum[GU];
  if constexpr (M == 2) {
    float acc[GU][5];
#pragma unroll
    for (int gi = 0; gi < GU; gi++)
#pragma unroll
      for (int i = 0; i < 5; i++) acc[gi][i] = 0.f;
#pragma unroll
    for (int dw = 0; dw < 8; dw++) {
      const int gi = (dw >> 1) * GU / 4;
      const uint32_t w = s0_dword(s.a, s.b, dw);
      const uint32_t* xq = xp + dw * 8;
      acc[gi][0] = dot2(w & 0x00030003u, xq[0], acc[gi][0]);
      acc[gi][1] = dot2(w & 0x000C000Cu, xq[1], acc[gi][1]);
      acc[gi][2] = dot2(w & 0x00300030u, xq[2], acc[gi][2]);
      acc[gi][3] = dot2(w & 0x00C000C0u, xq[3], acc[gi][3]);
      acc[gi][4] = dot2(w & 0x03000300u, xq[4], acc[gi][4]);
      const uint32_t t = w >> 6;
      acc[gi][2] = dot2(t & 0x00300030u, xq[5], acc[gi][2]);
      acc[gi][3] = dot2(t & 0x00C000C0u, xq[6], acc[gi][3]);
      acc[gi][4] = dot2(t & 0x03000300u, xq[7], acc[gi][4]);
    }
#pragma unroll
    for (int gi = 0; gi < GU; gi++)
      sum[gi] = acc[gi][0] * 0x1p24f + acc[gi][1] * 0x1p22f + acc[gi][2] * 0x1p20f +
                acc[gi][3] * 0x1p18f + acc[gi][4] * 0x1p16f;
  } else {
    float aA[GU], aB[GU], aC[GU];
#pragma unroll
    for (int gi = 0; gi < GU; gi++) { aA[gi] = 0.f; aB[gi] = 0.f; aC[gi] = 0.f; }
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const int gi = d * GU / 4;
      uint32_t ye, yo;
      const uint32_t p3 = s.pl[0][d];
      if constexpr (M >= 4) {
        pair_fields(p3, s.pl[1][d], ye, yo);
      } else {
        ye = (p3 << 1) & 0xAAAAAAAAu;
        yo = p3 & 0xAAAAAAAAu;
      }
      uint32_t ve = 0, vo = 0, we = 0, wo = 0;
      if constexpr (M >= 5) {
        const uint32_t p5 = s.pl[2][d];
        if constexpr (M >= 6) {
          pair_fields(p5, s.pl[3][d], ve, vo);
        } else {
          ve = (p5 << 1) & 0xAAAAAAAAu;
          vo = p5 & 0xAAAAAAAAu;
        }
        if constexpr (M >= 7) {
          const uint32_t p7 = s.pl[4][d];
          if constexpr (M >= 8) {
            pair_fields(p7, s.pl[5][d], we, wo);
          } else {
            we = (p7 << 1) & 0xAAAAAAAAu;
            wo = p7 & 0xAAAAAAAAu;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 2; e++) {
        uint32_t z[2];
        nibbles(s0_dword(s.a, s.b, 2 * d + e), e ? yo : ye, z[0], z[1]);
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const uint32_t* xq = xp + ((d * 2 + e) * 2 + h) * 4;
          const uint32_t zz = z[h], t = zz >> 8;
          aA[gi] = dot2(zz & 0x000F000Fu, xq[0], aA[gi]);
          aB[gi] = dot2(zz & 0x00F000F0u, xq[1], aB[gi]);
          aA[gi] = dot2(t & 0x000F000Fu, xq[2], aA[gi]);
          aB[gi] = dot2(t & 0x00F000F0u, xq[3], aB[gi]);
        }
        if constexpr (M >= 5) {
          uint32_t v[2];
          nibbles(e ? vo : ve, e ? wo : we, v[0], v[1]);
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const uint32_t* xq = xp + ((d * 2 + e) * 2 + h) * 4;
            const uint32_t zz = v[h], t = zz >> 8;
            aB[gi] = dot2(zz & 0x000F000Fu, xq[0], aB[gi]);
            aC[gi] = dot2(zz & 0x00F000F0u, xq[1], aC[gi]);
            aB[gi] = dot2(t & 0x000F000Fu, xq[2], aB[gi]);
            aC[gi] = dot2(t & 0x00F000F0u, xq[3], aC[gi]);
          }
        }
      }
    }
    // s_M sum(u_M x) = s * (aA 2^22 + aB 2^18 + aC 2^14) for every M >= 3.
#pragma unroll
    for (int gi = 0; gi < GU; gi++)
      sum[gi] = aA[gi] * 0x1p22f + aB[gi] * 0x1p18f + (M >= 5 ? aC[gi] * 0x1p14f : 0.f);
  }
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GU; gi++) {
    const float lo = h2f(s.meta[gi] & 0xffffu), st = h2f(s.meta[gi] >> 16);
    part += st * (sum[gi] - kM * sx[gi]) + lo * sx[gi];
  }
  return part;
}

// One step of a segmented inclusive scan inside 16-lane rows (DPP row_shr):
// add the value SH lanes down when it belongs to the same segment r.
template <int SH>
__device__ __forceinline__ float seg_step(float v, int r) {
  const int pv = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + SH, 0xf, 0xf, true);
  const int pr = __builtin_amdgcn_update_dpp(-1, r, 0x110 + SH, 0xf, 0xf, false);
  return pr == r ? v + __builtin_bit_cast(float, pv) : v;
}
// Carry across 16-lane rows: row_bcast:15 hands lane 15 of row 0/2 to rows
// 1/3 (row mask 0xa); row_bcast:31 hands lane 31 to rows 2 and 3 (mask 0xc).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float seg_bcast(float v, int r) {
  const int pv = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xf, false);
  const int pr = __builtin_amdgcn_update_dpp(-1, r, CTRL, ROWMASK, 0xf, false);
  return pr == r ? v + __builtin_bit_cast(float, pv) : v;
}
// Segmented inclusive scan over the 64 lanes of a wave (segment ids sorted by
// lane): afterwards the last lane of every segment holds the segment's sum.
__device__ __forceinline__ float seg_scan64(float v, int r) {
  v = seg_step<1>(v, r);
  v = seg_step<2>(v, r);
  v = seg_step<4>(v, r);
  v = seg_step<8>(v, r);
  v = seg_bcast<0x142, 0xa>(v, r);
  v = seg_bcast<0x143, 0xc>(v, r);
  return v;
}

// LDS column index of x: every 128-column tile is followed by 16 bytes of
// padding (conflict-free row reads in the correction phase).
__device__ __forceinline__ int xcol(int c) { return c + ((c >> 7) << 3); }

__device__ __forceinline__ uint64_t ld64side(rsrc_t r, uint32_t off) {
  const u32x2 v = ld64(r, off);
  return uint64_t(v[0]) | (uint64_t(v[1]) << 32);
}

template <int M, int GU, int D>
__global__ void __launch_bounds__(512) gemv_kernel(const GemvParams p) {
  extern __shared__ __align__(16) uint8_t lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);
  int32_t* rp_s = reinterpret_cast<int32_t*>(lds + p.lds_rp);
  uint32_t* meta_s = reinterpret_cast<uint32_t*>(lds + p.lds_meta);
  float* part_s = reinterpret_cast<float*>(lds + p.lds_part);
  float* corr_s = reinterpret_cast<float*>(lds + p.lds_corr);

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int r0 = blockIdx.x * p.RB;
  const int rip = tid / p.T;            // row slot within a pass
  const int t = tid - rip * p.T;        // tile column
  const bool act = rip < p.rpp;
  const int rows_here = min(p.RB, p.R - r0);

  const rsrc_t rA = mk(p.s0, p.chunk_bytes);
  const rsrc_t rB = mk(p.s0 + p.chunk_bytes, p.chunk_bytes);
  rsrc_t rP[M > 2 ? M - 2 : 1];
#pragma unroll
  for (int k = 0; k < M - 2; k++) rP[k] = mk(p.planes + uint64_t(k) * p.chunk_bytes, p.chunk_bytes);
  const rsrc_t rMeta = mk(p.meta, p.meta_bytes);
  const rsrc_t rX = mk(p.x, p.x_bytes);
  const rsrc_t rRp = mk(p.row_ptr, p.rp_bytes);
  const rsrc_t rSide = mk(p.side, p.side_bytes);

  // --- prologue.  Load order = arrival order: the workgroup's side-record
  //     range, this lane's x slice, x chunks and row_ptr for the LDS copies used
  //     at the end, then every pass of weights.  No barrier stands between the
  //     loads and the first pass.
  const uint32_t e0u = ld32(rRp, uint32_t(r0) * 4u);
  const uint32_t e1u = ld32(rRp, uint32_t(r0 + rows_here) * 4u);
  u32x4 xq[16];
  const uint32_t xbase = uint32_t(act ? t : 0) * 256u;
#pragma unroll
  for (int k = 0; k < 16; k++) xq[k] = ld128(rX, xbase + 16u * k);
  const int xchunks = p.C >> 3;
  u32x4 xv[kXChunks];
#pragma unroll
  for (int i = 0; i < kXChunks; i++) {
    const int ci = tid + i * nthr;
    xv[i] = ld128(rX, ci < xchunks ? uint32_t(ci) * 16u : kOOB);
  }
  uint32_t rpv[2];                       // row_ptr[r0 + j], j = tid, tid + nthr (<= rows_here)
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int j = tid + i * nthr;
    rpv[i] = ld32(rRp, j <= rows_here ? uint32_t(r0 + j) * 4u : kOOB);
  }
  __builtin_amdgcn_sched_barrier(0);
  Slot<M, GU> sl[D];
#pragma unroll
  for (int i = 0; i < D; i++) {          // slot by slot: pass i's loads complete first
    const int row = r0 + i * p.rpp + rip;
    issue(sl[i], rA, rB, rP, rMeta, uint32_t(row) * p.T + t, act && i < p.NP && row < p.R);
    __builtin_amdgcn_sched_barrier(0);
  }
  // LDS copies of x and row_ptr for the end (read after the loop's barrier).
  // The writes are unconditional (spare ones land in pad slots) so the loads
  // above are never sunk into a branch and waited on late.
#pragma unroll
  for (int i = 0; i < kXChunks; i++) {
    const int ci = tid + i * nthr;
    *reinterpret_cast<u32x4*>(xs + (ci < xchunks ? xcol(ci * 8) : xcol(p.C))) = xv[i];
  }
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int j = tid + i * nthr;
    rp_s[j <= rows_here ? j : p.RB + 1] = int32_t(rpv[i]);
  }
  const int e0 = int(e0u), e1 = int(e1u);

  // --- x slice of this lane's tile as permuted fp16 pairs; per-group sum(x).
  uint32_t xp[64];
  float sx[GU];
#pragma unroll
  for (int gi = 0; gi < GU; gi++) sx[gi] = 0.f;
#pragma unroll
  for (int d = 0; d < 4; d++) {
    uint32_t xr[64];
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const u32x4 v = xq[4 * d + q4];
      xr[16 * d + 4 * q4 + 0] = v[0]; xr[16 * d + 4 * q4 + 1] = v[1];
      xr[16 * d + 4 * q4 + 2] = v[2]; xr[16 * d + 4 * q4 + 3] = v[3];
    }
    const int gi = d * GU / 4;
#pragma unroll
    for (int i = 0; i < 16; i++) sx[gi] = dot2(xr[16 * d + i], kOneOne, sx[gi]);
    if constexpr (M == 2) {
#pragma unroll
      for (int e = 0; e < 2; e++)
#pragma unroll
        for (int i = 0; i < 8; i++)
          xp[(2 * d + e) * 8 + i] = pick(xr, 32 * d + 2 * i + e, 32 * d + 16 + 2 * i + e);
    } else {
#pragma unroll
      for (int e = 0; e < 2; e++)
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int m = 0; m < 4; m++)
            xp[((d * 2 + e) * 2 + h) * 4 + m] =
                pick(xr, 32 * d + 4 * m + 2 * h + e, 32 * d + 16 + 4 * m + 2 * h + e);
    }
  }

  // --- main loop.  A pass: the lane's tile partial; when a row's tiles are a
  //     power-of-two group of lanes inside one wave the row is summed at once
  //     with DPP and one value per row goes to LDS, otherwise one value per
  //     tile.  The slot is then reloaded with pass + D (out of range -> zeros,
  //     no traffic), which keeps every wait count path-independent.
  const int lane = tid & 63;
  uint64_t ent[kEntries];
  auto step_pass = [&](Slot<M, GU>& sl_i, int pass) {
    if (pass < p.NP) {
      float part = tile_partial<M, GU>(sl_i, xp, sx);
      if (p.red > 0) {
        // Every DPP step runs on all lanes (a lane reading a masked-off
        // neighbour would see 0); groups narrower than a 16-lane row then
        // keep the sum only where the source lane is in their own group.
        const int T = p.red;
        const int li = lane & (T - 1);
        float v;
        if (T >= 2) { v = seg_step<1>(part, 0); part = li >= 1 ? v : part; }
        if (T >= 4) { v = seg_step<2>(part, 0); part = li >= 2 ? v : part; }
        if (T >= 8) { v = seg_step<4>(part, 0); part = li >= 4 ? v : part; }
        if (T >= 16) part = seg_step<8>(part, 0);
        if (T >= 32) part = seg_bcast<0x142, 0xa>(part, T == 32 ? (lane >> 5) : 0);
        if (T >= 64) part = seg_bcast<0x143, 0xc>(part, 0);
        if (li == T - 1 && act) part_s[pass * p.rpp + rip] = part;
      } else if (act) {
        part_s[(pass * p.rpp + rip) * p.ppitch + t] = part;
      }
      if (act) {
        const int slot = pass * p.P + tid;
#pragma unroll
        for (int gi = 0; gi < GU; gi++) meta_s[slot * GU + gi] = sl_i.meta[gi];
      }
    }
    const int np = pass + D;
    const int row = r0 + np * p.rpp + rip;
    issue(sl_i, rA, rB, rP, rMeta, uint32_t(row) * p.T + t, act && np < p.NP && row < p.R);
  };
  // The first D passes in straight-line code; after the first, fetch this
  // workgroup's first side-record entries (one u64 each) for the end.
#pragma unroll
  for (int i = 0; i < D; i++) {
    step_pass(sl[i], i);
    if (i == 0) {
#pragma unroll
      for (int j = 0; j < kEntries; j++) {
        const int e = e0 + tid + j * nthr;
        ent[j] = ld64side(rSide, e < e1 ? uint32_t(e) * 8u : kOOB);
      }
    }
  }
  for (int pb = D; pb < p.NP; pb += D) {
#pragma unroll
    for (int i = 0; i < D; i++) step_pass(sl[i], pb + i);
  }
  __syncthreads();

  // --- side-record corrections (P - W_main) x_c, W_main = lo + s (q - 1/2 + 2^(1-M)),
  //     in chunks of kEntries * nthr entries in entry order.  Within each block
  //     of 64 consecutive entries (one wave) a segmented scan by row leaves, at
  //     the last entry of every row run, that run's sum; a row then adds one
  //     value per 64-entry block it touches.  Fixed order throughout.
  constexpr float kHeld = -0.5f + 1.0f / float(1 << (M - 1));
  const int chunk = kEntries * nthr;
  auto row_of = [&](uint64_t ev) -> int {   // row within the workgroup
    return int((uint32_t(ev >> 48) - uint32_t(r0)) & 0xffffu);
  };
  auto correction = [&](uint64_t ev) -> float {
    const int c = min(int(uint32_t(ev) & 0x3fffffffu), p.C - 1);
    const int q = int(uint32_t(ev) >> 30);
    const int rloc = min(row_of(ev), p.RB - 1);
    const int slot = (rloc / p.rpp) * p.P + (rloc % p.rpp) * p.T + (c >> 7);
    const int gi = (c & 127) / p.g;
    const uint32_t mw = meta_s[slot * GU + gi];
    const float lo = h2f(mw & 0xffffu), st = h2f(mw >> 16);
    const float wmain = lo + st * (float(q) + kHeld);
    return (h2f(uint32_t(ev >> 32) & 0xffffu) - wmain) * h2f(xs[xcol(c)]);
  };
  float rowc[2] = {0.f, 0.f};             // this thread's rows: tid and tid + nthr
  for (int ce = e0; ce < e1; ce += chunk) {
    if (ce > e0) {                        // rare: more entries than one prefetched chunk
      __syncthreads();                    // previous chunk consumed
#pragma unroll
      for (int j = 0; j < kEntries; j++) {
        const int e = ce + tid + j * nthr;
        ent[j] = ld64side(rSide, e < e1 ? uint32_t(e) * 8u : kOOB);
      }
    }
#pragma unroll
    for (int j = 0; j < kEntries; j++) {
      const bool ok = ce + tid + j * nthr < e1;
      corr_s[tid + j * nthr] = seg_scan64(correction(ent[j]), ok ? row_of(ent[j]) : p.RB);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int i = tid + k * nthr;
      if (i < rows_here) {
        const int a = max(rp_s[i], ce) - ce, b = min(rp_s[i + 1], ce + chunk) - ce;
        for (int q = a; q < b; q = (q | 63) + 1) rowc[k] += corr_s[min(b, (q | 63) + 1) - 1];
      }
    }
  }

  // --- row sums: one thread per row.
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int i = tid + k * nthr;
    if (i < rows_here) {
      float acc;
      if (p.red > 0) {
        acc = part_s[i];
      } else {
        const float* pr = part_s + i * p.ppitch;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        int tt = 0;
        for (; tt + 4 <= p.T; tt += 4) { a0 += pr[tt]; a1 += pr[tt + 1]; a2 += pr[tt + 2]; a3 += pr[tt + 3]; }
        for (; tt < p.T; tt++) a0 += pr[tt];
        acc = (a0 + a1) + (a2 + a3);
      }
      p.y[r0 + i] = acc + rowc[k];
    }
  }
}

// Code dump: one thread per tile writes the 128 codes u_M of its tile.
struct CodesParams {
  const uint8_t* s0;
  const uint8_t* planes;
  uint8_t* codes;
  uint32_t chunk_bytes;
  int32_t T, C;
  int64_t tiles;
};

template <int M>
__global__ void __launch_bounds__(256) codes_kernel(const CodesParams p) {
  const int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (u >= p.tiles) return;
  const rsrc_t rA = mk(p.s0, p.chunk_bytes), rB = mk(p.s0 + p.chunk_bytes, p.chunk_bytes);
  const uint32_t off = uint32_t(u) * 16u;
  const u32x4 a = ld128(rA, off), b = ld128(rB, off);
  u32x4 pl[M > 2 ? M - 2 : 1];
#pragma unroll
  for (int k = 0; k < M - 2; k++) pl[k] = ld128(mk(p.planes + uint64_t(k) * p.chunk_bytes, p.chunk_bytes), off);
  uint32_t out[32];  // out[8d + m] = codes of columns 32d + 4m .. 32d + 4m + 3
#pragma unroll
  for (int d = 0; d < 4; d++) {
    if constexpr (M == 2) {
#pragma unroll
      for (int m = 0; m < 8; m++) {
        uint32_t o = 0;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
          const uint32_t w = s0_dword(a, b, 2 * d + (bb & 1));
          o |= ((w >> (2 * (2 * m + (bb >> 1)))) & 3u) << (8 * bb);
        }
        out[8 * d + m] = o;
      }
    } else {
      uint32_t ye, yo;
      if constexpr (M >= 4) {
        pair_fields(pl[0][d], pl[1][d], ye, yo);
      } else {
        ye = (pl[0][d] << 1) & 0xAAAAAAAAu;
        yo = pl[0][d] & 0xAAAAAAAAu;
      }
      uint32_t ve = 0, vo = 0, we = 0, wo = 0;
      if constexpr (M >= 5) {
        if constexpr (M >= 6) pair_fields(pl[2][d], pl[3][d], ve, vo);
        else { ve = (pl[2][d] << 1) & 0xAAAAAAAAu; vo = pl[2][d] & 0xAAAAAAAAu; }
        if constexpr (M >= 7) {
          if constexpr (M >= 8) pair_fields(pl[4][d], pl[5][d], we, wo);
          else { we = (pl[4][d] << 1) & 0xAAAAAAAAu; wo = pl[4][d] & 0xAAAAAAAAu; }
        }
      }
      uint32_t z[2][2], v[2][2];
#pragma unroll
      for (int e = 0; e < 2; e++) {
        nibbles(s0_dword(a, b, 2 * d + e), e ? yo : ye, z[e][0], z[e][1]);
        nibbles(e ? vo : ve, e ? wo : we, v[e][0], v[e][1]);
      }
#pragma unroll
      for (int m = 0; m < 8; m++) {
        uint32_t o = 0;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
          const int e = bb & 1, h = bb >> 1;
          const uint32_t n0 = (z[e][h] >> (4 * m)) & 15u;   // q b3 b4 (zeros below a short read)
          uint32_t code;
          if constexpr (M == 3) code = n0 >> 1;
          else if constexpr (M == 4) code = n0;
          else code = (n0 << (M - 4)) | (((v[e][h] >> (4 * m)) & 15u) >> (8 - M));
          o |= code << (8 * bb);
        }
        out[8 * d + m] = o;
      }
    }
  }
  const int64_t row = u / p.T, tc = u % p.T;
  u32x4* dst = reinterpret_cast<u32x4*>(p.codes + row * p.C + tc * 128);
#pragma unroll
  for (int i = 0; i < 8; i++) {
    u32x4 v;
    v[0] = out[4 * i]; v[1] = out[4 * i + 1]; v[2] = out[4 * i + 2]; v[3] = out[4 * i + 3];
    dst[i] = v;
  }
}

}  // namespace dev

// ------------------------------------------------------------- dispatch ----
struct LaunchCfg {
  int waves, rpp, NP, RB, grid, L;
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

static int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

constexpr size_t kLdsBudget = 64 * 1024;
// Passes of loads in flight per precision (bounded by the VGPRs of a slot:
// 8 + 4 (M - 2) + pairs dwords).
constexpr int kDepth[9] = {0, 0, 8, 4, 4, 2, 2, 2, 2};
constexpr int kMaxWaves = 8;  // matches __launch_bounds__(512) of the GEMV kernel

// LDS carve-up of one workgroup: padded x (plus one spare 16-byte slot),
// row_ptr of its rows (plus a spare slot), group pairs of every tile it owns,
// row (or tile) partials, and one chunk of scanned side-record corrections.
static size_t lds_layout(int C, int GU, int nthr, int NP, int rpp, int P, int T, bool red,
                         dev::GemvParams* prm) {
  const size_t units = size_t(NP) * P;
  const int RB = NP * rpp;
  size_t o = size_t(C) * 2 + size_t(C / kTileCols) * 16 + 16;
  if (prm) prm->lds_rp = uint32_t(o);
  o += size_t(RB + 2) * 4;
  o = (o + 15) & ~size_t(15);
  if (prm) prm->lds_meta = uint32_t(o);
  o += units * 4 * GU;
  if (prm) prm->lds_part = uint32_t(o);
  o += red ? size_t(RB) * 4 : size_t(RB) * (T + 1) * 4;
  o = (o + 15) & ~size_t(15);
  if (prm) prm->lds_corr = uint32_t(o);
  o += size_t(dev::kEntries) * nthr * 4;
  return o;
}

// Rows are summed inside the loop when a row's tiles form a power-of-two group
// of lanes within one wave.
static bool row_reduce(int T) { return T <= 64 && (T & (T - 1)) == 0; }

// Launch shape for one GEMV: k waves per workgroup, rpp rows side by side
// (rpp * tiles_per_row lanes busy), NP passes per workgroup.  Among the shapes
// that fit LDS, pick the lowest estimated cost on the busiest CU: rounds of
// workgroups x (passes + 2 of overhead) x lanes, a third more when not all
// passes fit in flight (NP > depth); ties go to more waves.  STAGQ_WAVES / STAGQ_NP
// override the choice (tuning).
static bool plan_gemv(const ImageHeader& h, int GU, int depth, LaunchCfg* c) {
  const int T = h.cols / kTileCols;
  const int R = h.rows;
  const int cus = device_cus();
  const int kmin = std::max(std::max((T + 63) / 64, 1),
                            (h.cols / 8 + dev::kXChunks * 64 - 1) / (dev::kXChunks * 64));
  const int k_env = env_int("STAGQ_WAVES", 0), np_env = env_int("STAGQ_NP", 0);
  bool found = false;
  long best_work = 0;
  int best_k = 0, best_np = 0;
  bool best_fly = false;
  for (int k = kmin; k <= kMaxWaves; k++) {
    if (k_env && k != k_env) continue;
    const int nthr = 64 * k, rpp = nthr / T;
    if (rpp < 1) continue;
    const double util = double(rpp * T) / nthr;
    if (util < 0.85 && !k_env) continue;
    const int passes = (R + rpp - 1) / rpp;
    for (int np = 1; np <= passes; np++) {
      if (np_env && np != np_env) continue;
      if (lds_layout(h.cols, GU, nthr, np, rpp, rpp * T, T, row_reduce(T), nullptr) > kLdsBudget ||
          np * rpp + 1 > 2 * nthr)
        break;
      const int grid = (passes + np - 1) / np;
      const bool fly = np <= depth;
      // lane-passes on the busiest CU, each workgroup paying about two passes
      // of prologue and epilogue; a third more when passes must wait for slots
      const long work = long((grid + cus - 1) / cus) * (np + 2) * nthr * (fly ? 3 : 4);
      const bool better = !found || work < best_work ||
                          (work == best_work && fly && !best_fly) ||
                          (work == best_work && fly == best_fly && k > best_k);
      if (better) { found = true; best_work = work; best_k = k; best_np = np; best_fly = fly; }
    }
  }
  if (!found) return false;
  const int k = best_k, NP = best_np;
  const int nthr = 64 * k, rpp = nthr / T, P = rpp * T;
  const int RB = NP * rpp;
  c->waves = k; c->rpp = rpp; c->NP = NP; c->RB = RB;
  c->grid = (R + RB - 1) / RB;
  c->L = 0;
  const bool red = row_reduce(T);
  c->lds = lds_layout(h.cols, GU, nthr, NP, rpp, P, T, red, &c->prm);
  c->prm.R = R; c->prm.C = h.cols; c->prm.T = T; c->prm.g = h.group; c->prm.rpp = rpp;
  c->prm.P = P; c->prm.NP = NP; c->prm.RB = RB;
  c->prm.red = red ? T : 0;
  c->prm.ppitch = T + 1;
  return true;
}

template <int M, int GU, int D>
static hipError_t launch_gemv(const LaunchCfg& c, hipStream_t st) {
  hipLaunchKernelGGL((dev::gemv_kernel<M, GU, D>), dim3(c.grid), dim3(64 * c.waves), c.lds, st, c.prm);
  return hipGetLastError();
}

template <int M, int GU>
static hipError_t launch_gemv_d(const LaunchCfg& c, hipStream_t st) {
  return launch_gemv<M, GU, kDepth[M]>(c, st);
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
  for (int b = 2; b <= h->hdr.nbits; b++) out->bytes_read[b] = bytes_read(h->hdr, b);
  return STAGQ_OK;
}

void stagq_destroy(stagq_handle h) { delete h; }

int stagq_gemv(stagq_handle h, const void* x, float* y, int bits, void* hip_stream) {
  if (!h) return STAGQ_EINVAL;
  const ImageHeader& H = h->hdr;
  if (bits < 2 || bits > H.nbits) return STAGQ_EBITS;
  if (H.rows == 0) return STAGQ_OK;  // nothing to compute; y may be empty
  if (!x || !y) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 4) return STAGQ_EALIGN;
  const int GU = kTileCols / H.group;
  LaunchCfg c;
  if (!plan_gemv(H, GU, kDepth[bits], &c)) return STAGQ_ESHAPE;
  const uint8_t* b = h->dev;
  c.prm.s0 = b + H.off_s0;
  c.prm.planes = b + H.off_planes;
  c.prm.meta = b + H.off_meta;
  c.prm.row_ptr = b + H.off_rowptr;
  c.prm.side = b + H.off_side;
  c.prm.x = static_cast<const uint8_t*>(x);
  c.prm.y = y;
  c.prm.chunk_bytes = uint32_t(H.bytes_s0_chunk);
  c.prm.meta_bytes = uint32_t(H.bytes_meta);
  c.prm.side_bytes = uint32_t(H.nnz * 8);
  c.prm.rp_bytes = uint32_t((H.rows + 1) * 4);
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

int stagq_plan_gemv(int32_t rows, int32_t cols, int32_t group, int32_t nbits, int bits,
                    int32_t* out) {
  if (!out) return STAGQ_EINVAL;
  ImageHeader H;
  if (!layout(rows, cols, group, nbits, 0, &H)) return STAGQ_ESHAPE;
  if (bits < 2 || bits > nbits) return STAGQ_EBITS;
  LaunchCfg c;
  if (!plan_gemv(H, kTileCols / group, kDepth[bits], &c)) return STAGQ_ESHAPE;
  out[0] = c.grid; out[1] = 64 * c.waves; out[2] = c.rpp; out[3] = c.NP; out[4] = c.RB;
  out[5] = int32_t(c.lds); out[6] = c.L; out[7] = kDepth[bits];
  return STAGQ_OK;
}

int stagq_decode_codes(stagq_handle h, int bits, uint8_t* codes, void* hip_stream) {
  if (!h) return STAGQ_EINVAL;
  const ImageHeader& H = h->hdr;
  if (bits < 2 || bits > H.nbits) return STAGQ_EBITS;
  if (H.tiles == 0) return STAGQ_OK;
  if (!codes) return STAGQ_EINVAL;
  if (reinterpret_cast<uintptr_t>(codes) % 16) return STAGQ_EALIGN;
  dev::CodesParams p;
  p.s0 = h->dev + H.off_s0;
  p.planes = h->dev + H.off_planes;
  p.codes = codes;
  p.chunk_bytes = uint32_t(H.bytes_s0_chunk);
  p.T = H.cols / kTileCols;
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
