// MFMA, LDS and cross-lane building blocks shared by the bf16 attention kernels.
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (A: 32x16, B: 16x32, C: 32x32 fp32)
// for lane l, g = l / 32, c = l % 32:
//   A: 8 bf16  A[c][8g .. 8g+7]
//   B: 8 bf16  B[8g .. 8g+7][c]
//   C: 16 fp32 C[8i + 4g + j][c] at element 4i + j
// ds_read_b64_tr_b16 (gfx950) works on groups of 16 lanes: if lane j = 4r + s
// of a group reads the 4 bf16 M[j][0..3], lane i of the group receives
// (M[i/4][i%4], M[4 + i/4][i%4], M[8 + i/4][i%4], M[12 + i/4][i%4]).  Four lanes
// reading 4 consecutive values each of row r therefore hand lane i the values of
// 4 rows at one column: a transposed operand read from a row-major tile.
#pragma once

#include "sta_common.h"

namespace sta {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row-major bf16 tiles in LDS with D/8 16-byte chunks per row; chunk c of row r
// is stored at chunk position c ^ swz<D>(r).  The gfx950 LDS serves 256 bytes
// per clock (64 banks): a 16-byte-per-lane read is conflict-free when each 16
// consecutive lanes touch 16 distinct 16-byte bank groups of a 256-byte line.
//   D = 128 (256-byte rows): 16 consecutive rows at one chunk -> 16 distinct
//     positions (K operand reads); rows 4m..4m+3 x 4 adjacent chunks -> 16
//     distinct positions (transposed V operand reads).
//   D = 64 (128-byte rows, two rows per line): the same two properties with the
//     row parity supplying the line half.
template <int D>
__device__ __forceinline__ uint32_t swz(uint32_t r) {
  if constexpr (D == 128) {
    return ((r & 3u) << 2) | ((r >> 2) & 3u);
  } else {
    return (((r >> 1) & 1u) << 2) | ((r >> 2) & 3u);
  }
}

template <int D>
__device__ __forceinline__ uint32_t tile_off(uint32_t r, uint32_t chunk) {  // bytes
  return r * (D * 2) + ((chunk ^ swz<D>(r)) << 4);
}

__device__ __forceinline__ u32x4 lds_read16(const char* base, uint32_t off) {
  return *(const u32x4*)(base + off);
}

// Transposed 8-byte read (see the layout note above).
__device__ __forceinline__ s16x4 lds_read_tr(const char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off));
}

__device__ __forceinline__ bf16x8 join_tr(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l writes bytes
// [16 l, 16 l + 16) of the 1 KiB LDS segment starting at lds (wave-uniform).
__device__ __forceinline__ void dma16(const void* gsrc, void* lds) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_ptr_t)lds, 16, 0, 0);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Wait until at most N vector-memory operations (here: DMA copies) of this
// wave are still in flight (s_waitcnt vmcnt(N), expcnt and lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_dma_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait for this wave's LDS accesses (s_waitcnt lgkmcnt(0), vmcnt untouched).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Workgroup barrier for the LDS pipelines.  The only LDS writes the kernels
// make are DMA copies, each wave waits for its own with wait_dma*() first, so
// the barrier needs no memory fence (__syncthreads() would also drain every
// copy still in flight).  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Padding mask of one 32-row block: bit r is set when intra-tile position
// row0 + r of tile (a0, a1, a2) holds a real token.  The same value in every
// lane (a ballot; every lane must call it).
__device__ __forceinline__ uint32_t block_real_mask(int a0, int a1, int a2, int row0,
                                                    const Geometry& g, int lane) {
  const bool real = token_real(a0, a1, a2, row0 + (lane & 31), g);
  return (uint32_t)__ballot(real);
}

// The block mask seen from an MFMA accumulator whose element 4i + j in lane l
// holds row 8i + 4(l / 32) + j: bit 8i + j of the result belongs to element
// 4i + j (test it with elem_real).
__device__ __forceinline__ uint32_t lane_bits(uint32_t block_mask, int lane) {
  return block_mask >> (4 * (lane >> 5));
}

__device__ __forceinline__ bool elem_real(uint32_t bits, int e) {
  return (bits >> (8 * (e >> 2) + (e & 3))) & 1u;
}

// Position (t, h, w) inside a partial tile of index c in its compacted order
// (the tile's real tokens in (t, h, w) order, padding positions left out),
// e1 and e2 the tile's real extents along h and w and inv1, inv2 their fp32
// reciprocals.  Exact for c < 2^20: (c + 0.5) / e then lies at least 2^-21
// (relative) away from any integer, beyond the reciprocal's error.
struct TilePos {
  uint32_t t, h, w;
};
__device__ __forceinline__ TilePos split_compact(uint32_t c, int e1, int e2, float inv1, float inv2) {
  const uint32_t tr = (uint32_t)(((float)c + 0.5f) * inv2);  // tile row (t, h)
  const uint32_t ct = (uint32_t)(((float)tr + 0.5f) * inv1);
  return {ct, tr - ct * (uint32_t)e1, c - tr * (uint32_t)e2};
}

// x combined with the value of lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float xsum32(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Copies of K and V blocks [ROWS x D] into LDS tiles in the swizzled layout
// with 16-byte DMA.  The 1 KiB segments of each tile are dealt round-robin
// over the NW waves of the workgroup; the source offset of each lane's 16
// bytes inside a block and the wave's LDS segments do not change from block
// to block, so they are worked out once and an issue costs one scalar base per
// tensor (the loads use the scalar-base + 32-bit lane-offset addressing form).
// wave_u must be the wave index held uniformly (readfirstlane).
template <int D, int ROWS, int NW>
struct KvDma {
  static constexpr int RPS = 1024 / (D * 2);  // rows per 1 KiB segment
  static constexpr int SEGS = ROWS / RPS;     // segments per tile
  static_assert(ROWS % RPS == 0 && SEGS % NW == 0, "segments must split evenly over waves");
  static constexpr int PT = SEGS / NW;        // segments per wave per tile
  static constexpr int PER = 2 * PT;          // copies per wave per issue
  uint32_t goff[PT];
  int wave_u;
  __device__ __forceinline__ KvDma(int wave_uniform, int lane) : wave_u(wave_uniform) {
    constexpr int CPR = D / 8;  // chunks per row
    const int rin = lane / CPR, p = lane % CPR;
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const int r = (wave_u + e * NW) * RPS + rin;
      goff[e] = (uint32_t)(r * D + ((p ^ (int)swz<D>(r)) * 8)) * 2u;
    }
  }
  // Lane offset e, opaque to the optimiser at each use: otherwise it hoists
  // the loop-invariant sum of tensor base and lane offset into a 64-bit
  // register pair and adds each block's row offset with 64-bit vector adds,
  // where the scalar-base form needs none.
  __device__ __forceinline__ uint32_t lane_off(int e) const {
    uint32_t o = goff[e];
    asm volatile("" : "+v"(o));
    return o;
  }
  // Rows [row0, row0 + ROWS) of kg and vg into the tiles kl and vl.
  __device__ __forceinline__ void issue(const uint16_t* kg, const uint16_t* vg, size_t row0, char* kl,
                                        char* vl) const {
    const char* kbase = (const char*)(kg + row0 * D);
    const char* vbase = (const char*)(vg + row0 * D);
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const int seg = wave_u + e * NW;
      const uint32_t o = lane_off(e);
      dma16(kbase + o, kl + seg * 1024);
      dma16(vbase + o, vl + seg * 1024);
    }
  }
  // The same block gathered from a raster-order sequence, addressed from a
  // key tile's origin row (origin_row, scalar): seg_off[e] is the raster
  // offset of the first of the RPS rows of segment wave + e * NW from that
  // origin (scalar, never negative; those rows must be consecutive in raster
  // order).  One scalar base per tensor and a 32-bit lane offset per segment.
  __device__ __forceinline__ void issue_rows_origin(const uint16_t* kg, const uint16_t* vg,
                                                    uint32_t origin_row, const uint32_t (&seg_off)[PT],
                                                    char* kl, char* vl) const {
    const char* kbase = (const char*)(kg + (size_t)origin_row * D);
    const char* vbase = (const char*)(vg + (size_t)origin_row * D);
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const int seg = wave_u + e * NW;
      const uint32_t in_seg = goff[e] - (uint32_t)(seg * RPS * D * 2);
      const uint32_t off = seg_off[e] * (uint32_t)(D * 2) + in_seg;
      dma16(kbase + off, kl + seg * 1024);
      dma16(vbase + off, vl + seg * 1024);
    }
  }
  // Row of the block that the lane's copy of segment e fills (worked out at
  // each use, like lane_off, rather than held in a register).
  __device__ __forceinline__ uint32_t row_in_block(int e, int lane) const {
    uint32_t l = (uint32_t)lane;
    asm volatile("" : "+v"(l));
    return (uint32_t)((wave_u + e * NW) * RPS) + l / (uint32_t)(D / 8);
  }
  // The same block gathered row by row (a key tile that holds padding, its
  // real keys compacted): the lane's row of segment e is row_off[e] rows past
  // origin_row (scalar).  Lanes whose row is padding (real[e] false) copy 16
  // bytes of the origin row itself, a real row, so no read leaves the tensor;
  // the attention masks those keys.
  __device__ __forceinline__ void issue_rows_gather(const uint16_t* kg, const uint16_t* vg,
                                                    uint32_t origin_row, const uint32_t (&row_off)[PT],
                                                    const bool (&real)[PT], char* kl, char* vl) const {
    const char* kbase = (const char*)(kg + (size_t)origin_row * D);
    const char* vbase = (const char*)(vg + (size_t)origin_row * D);
#pragma unroll
    for (int e = 0; e < PT; ++e) {
      const int seg = wave_u + e * NW;
      const uint32_t off = (real[e] ? row_off[e] * (uint32_t)(D * 2) : 0u) + in_row(e);
      dma16(kbase + off, kl + seg * 1024);
      dma16(vbase + off, vl + seg * 1024);
    }
  }
  // The K block alone (PT copies per wave).
  __device__ __forceinline__ void issue_k(const uint16_t* kg, size_t row0, char* kl) const {
    const char* kbase = (const char*)(kg + row0 * D);
#pragma unroll
    for (int e = 0; e < PT; ++e) dma16(kbase + lane_off(e), kl + (wave_u + e * NW) * 1024);
  }
  // The K block alone, gathered row by row as in issue_rows_gather.
  __device__ __forceinline__ void issue_k_gather(const uint16_t* kg, uint32_t origin_row,
                                                 const uint32_t (&row_off)[PT], const bool (&real)[PT],
                                                 char* kl) const {
    const char* kbase = (const char*)(kg + (size_t)origin_row * D);
#pragma unroll
    for (int e = 0; e < PT; ++e)
      dma16(kbase + (real[e] ? row_off[e] * (uint32_t)(D * 2) : 0u) + in_row(e), kl + (wave_u + e * NW) * 1024);
  }
  // The lane's (swizzled) 16-byte chunk inside its row of segment e.
  __device__ __forceinline__ uint32_t in_row(int e) const {
    return lane_off(e) % (uint32_t)(D * 2);
  }
};

// A/B operand fragments of a row-major [32 x D] tile (rows = keys or
// queries): lane l holds 8 consecutive d of row l % 32 for each 16-wide k-step.
template <int D>
__device__ __forceinline__ void read_rows(const char* tl, bf16x8 (&f)[D / 16], int grp, int c32) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    f[ks] = as_bf16x8(lds_read16(tl, tile_off<D>(c32, ks * 2 + grp)));
}

// Transposed fragments of the same tile, [d][row] with the row order of the
// 32x32 accumulator: lane i of each 16-lane group takes d = dt*32 + 16h + i
// and rows (16s + 4g + r) and (16s + 8 + 4g + r), r = 0..3.  Element e of
// fragment [dt][s] is row 16s + 8(e/4) + 4g + e%4, which is the row held in
// element 8s + e of a 32x32 accumulator whose lane owns column l % 32.
template <int D>
__device__ __forceinline__ void read_cols(const char* tl, bf16x8 (&f)[D / 32][2], int lane) {
  const int grp = lane >> 5, l16 = lane & 15, h = (lane >> 4) & 1;
  const int vr = grp * 4 + (l16 >> 2);
  const int vc = l16 & 3;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int d = dt * 32 + 16 * h + 4 * vc;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r0 = 16 * s + vr;
      const s16x4 lo = lds_read_tr(tl, tile_off<D>(r0, d >> 3) + (d & 4) * 2);
      const s16x4 hi = lds_read_tr(tl, tile_off<D>(r0 + 8, d >> 3) + (d & 4) * 2);
      f[dt][s] = join_tr(lo, hi);
    }
  }
}

}  // namespace sta
