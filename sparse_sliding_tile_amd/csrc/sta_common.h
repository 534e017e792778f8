// Shared definitions for the libsta HIP kernels (gfx950).
//
// The tile-window rule lives here, once, as a host+device function: the
// forward, backward and pair-export kernels and the host-side pair list all
// call window_start() so they cannot disagree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sta.h"

#define STA_HD __host__ __device__ __forceinline__

namespace sta {

// ---------------------------------------------------------------------------
// Window rule ("Sliding Tile Attention", arXiv 2502.04507 summary page, method
// details: a query tile attends to a local window of whole tiles).  Along one
// dimension with n tiles and a window of w tiles, w' = min(w, n) and the window
// of query tile q is [s, s + w') with s = clamp(q - floor(w'/2), 0, n - w').
// ---------------------------------------------------------------------------
STA_HD int window_width(int w, int n) { return w < n ? w : n; }

STA_HD int window_start(int q, int wp, int n) {
  int s = q - wp / 2;
  s = s < 0 ? 0 : s;
  return s > n - wp ? n - wp : s;
}

// Query tiles whose window holds key tile k, along one dimension: since
// window_start is non-decreasing in q, they form one interval [lo, hi].
STA_HD void window_transpose(int k, int wp, int n, int* lo, int* hi) {
  int a = 0;
  while (a < n && window_start(a, wp, n) + wp <= k) ++a;
  int b = n - 1;
  while (b >= 0 && window_start(b, wp, n) > k) --b;
  *lo = a;
  *hi = b;
}

// ---------------------------------------------------------------------------
// Unsigned division by a run-time invariant d >= 1 for 0 <= n < 2^31, with a
// multiply-high and a shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994): l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l.
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.l = l;
  f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  return f;
}

STA_HD uint32_t fdiv(uint32_t n, FastDiv f) {
#ifdef __HIP_DEVICE_COMPILE__
  uint32_t hi = __umulhi(f.m, n);
#else
  uint32_t hi = (uint32_t)(((uint64_t)f.m * n) >> 32);
#endif
  return (hi + n) >> f.l;
}

// Per-launch geometry, passed by value in the kernel arguments.
struct Geometry {
  int T, H, W;     // latent (real tokens)
  int t, h, w;     // tile
  int n0, n1, n2;  // tile grid, ceil(latent / tile) per dimension
  int L;           // tokens per tile
  int S;           // tile-major rows per (b, head): n0 * n1 * n2 * L
  int Sr;          // raster rows per (b, head): T * H * W
  int ntiles;      // n0 * n1 * n2
  int padded;      // 1 when the latent is not a whole number of tiles
  FastDiv fw, fhw; // division by w and by h * w (intra-tile coordinates)
};

// Padding with masking ("Fast Video Generation with Sliding Tile Attention",
// OpenReview rebuttal, answer on input resolution): a latent that is not a
// whole number of tiles is padded up to the next multiple in each dimension.
// Tile a then holds real tokens only in the box of intra-tile coordinates
// [0, ext) per dimension, ext = min(tile, latent - a * tile); the other
// positions are padding: never keys, and their output rows are zero.
STA_HD int tile_ext(int a, int tile, int latent) {
  const int e = latent - a * tile;
  return e < tile ? e : tile;
}

STA_HD bool tile_partial(int a0, int a1, int a2, const Geometry& g) {
  return tile_ext(a0, g.t, g.T) < g.t || tile_ext(a1, g.h, g.H) < g.h ||
         tile_ext(a2, g.w, g.W) < g.w;
}

// Whether intra-tile position i (raster order inside the tile) of tile
// (a0, a1, a2) holds a real token.
STA_HD bool token_real(int a0, int a1, int a2, int i, const Geometry& g) {
  const uint32_t i01 = fdiv((uint32_t)i, g.fw), i0 = fdiv((uint32_t)i, g.fhw);
  const int i2 = i - (int)i01 * g.w, i1 = (int)i01 - (int)i0 * g.h;
  return (int)i0 < tile_ext(a0, g.t, g.T) && i1 < tile_ext(a1, g.h, g.H) && i2 < tile_ext(a2, g.w, g.W);
}

// Largest tile count along one grid dimension: clamped window widths are held
// in 16 bits (HeadTable, MassArgs).
constexpr int64_t kMaxGridTiles = 65535;

// Per-head windows, already clamped to the grid (w'), plus a launch order of
// the heads (heaviest first) for load balance.  Lives in the kernel arguments,
// so each launch carries its own copy.
struct HeadTable {
  uint16_t wp[STA_MAX_HEADS][3];
  uint8_t order[STA_MAX_HEADS];
};

// ---------------------------------------------------------------------------
// Vector types for MFMA operands and 16-byte memory traffic.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace sta
