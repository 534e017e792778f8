// Tile reorder / unreorder and the tile-pair export.
//
// Reorder ("Sliding Tile Attention", arXiv 2502.04507 summary page, method
// details: the latent is cut into non-overlapping space-time tiles and every
// tile is made one contiguous run of the sequence).  A bit-exact gather/scatter
// bound by HBM bandwidth: one workgroup moves one tile of one (batch, head); the
// w tokens of a tile row are contiguous in both orders, so every wavefront reads
// and writes whole token rows with 16-byte accesses.  A latent that is not a
// whole number of tiles is padded with masking (OpenReview rebuttal, answer on
// input resolution): the reorder writes zero rows at padding positions of the
// tile-major tensor and the unreorder skips them.
#include "kernels.h"

namespace sta {

template <int G>
struct Chunk;
template <>
struct Chunk<16> { typedef u32x4 type; };
template <>
struct Chunk<8> { typedef u32x2 type; };
template <>
struct Chunk<4> { typedef uint32_t type; };
template <>
struct Chunk<2> { typedef uint16_t type; };

// One workgroup per (tile, b*Hh).  Each thread moves G-byte chunks; U chunks
// are loaded before any is stored so several loads are in flight per thread.
template <int G, int U>
__global__ __launch_bounds__(256) void tile_copy_kernel(const char* __restrict__ src,
                                                        char* __restrict__ dst, Geometry g,
                                                        uint32_t row_bytes, FastDiv fd_units,
                                                        FastDiv fd_w, FastDiv fd_h,
                                                        int to_tile_major) {
  typedef typename Chunk<G>::type V;
  const uint32_t tile = blockIdx.x % (uint32_t)g.ntiles;
  const uint64_t bh = blockIdx.x / (uint32_t)g.ntiles;
  const uint32_t a2 = tile % g.n2;
  const uint32_t a01 = tile / g.n2;
  const uint32_t a1 = a01 % g.n1;
  const uint32_t a0 = a01 / g.n1;
  const uint32_t units = (uint32_t)g.L * fd_units.d;
  const uint64_t rbase = bh * (uint64_t)g.Sr * row_bytes;  // raster tensor
  const uint64_t tbase = bh * (uint64_t)g.S * row_bytes;   // tile-major tensor
  const int e0 = tile_ext(a0, g.t, g.T), e1 = tile_ext(a1, g.h, g.H), e2 = tile_ext(a2, g.w, g.W);

  for (uint32_t u0 = threadIdx.x; u0 < units; u0 += 256 * U) {
    V val[U];
    uint64_t doff[U];
    bool store[U];
#pragma unroll
    for (int e = 0; e < U; ++e) {
      const uint32_t u = u0 + e * 256;
      store[e] = false;
      if (u < units) {
        const uint32_t i = fdiv(u, fd_units);          // token inside the tile
        const uint32_t c = u - i * fd_units.d;         // chunk inside the token row
        const uint32_t i01 = fdiv(i, fd_w);
        const uint32_t i2 = i - i01 * g.w;
        const uint32_t i0 = fdiv(i01, fd_h);
        const uint32_t i1 = i01 - i0 * g.h;
        const bool real = (int)i0 < e0 && (int)i1 < e1 && (int)i2 < e2;
        const uint64_t raster =
            ((uint64_t)(a0 * g.t + i0) * g.H + (a1 * g.h + i1)) * g.W + (a2 * g.w + i2);
        const uint64_t tm = (uint64_t)tile * g.L + i;
        const uint64_t roff = rbase + raster * row_bytes + (uint64_t)c * G;
        const uint64_t toff = tbase + tm * row_bytes + (uint64_t)c * G;
        doff[e] = to_tile_major ? toff : roff;
        store[e] = real || to_tile_major;  // padding: zero in tile-major, nothing in raster
        val[e] = V{};
        if (real) val[e] = __builtin_nontemporal_load((const V*)(src + (to_tile_major ? roff : toff)));
      }
    }
#pragma unroll
    for (int e = 0; e < U; ++e) {
      if (store[e]) __builtin_nontemporal_store(val[e], (V*)(dst + doff[e]));
    }
  }
}

hipError_t launch_tile_copy(const void* src, void* dst, int64_t BH, int64_t row_bytes,
                            const Geometry& g, bool to_tile_major, hipStream_t stream) {
  int G = 16;
  while (row_bytes % G) G >>= 1;
  const uint32_t units_per_row = (uint32_t)(row_bytes / G);
  const FastDiv fu = make_fastdiv(units_per_row), fw = make_fastdiv(g.w), fh = make_fastdiv(g.h);
  const dim3 grid((uint32_t)(g.ntiles * BH));
  const int flag = to_tile_major ? 1 : 0;
  const char* s = (const char*)src;
  char* d = (char*)dst;
  switch (G) {
    case 16:
      hipLaunchKernelGGL((tile_copy_kernel<16, 4>), grid, dim3(256), 0, stream, s, d, g,
                         (uint32_t)row_bytes, fu, fw, fh, flag);
      break;
    case 8:
      hipLaunchKernelGGL((tile_copy_kernel<8, 4>), grid, dim3(256), 0, stream, s, d, g,
                         (uint32_t)row_bytes, fu, fw, fh, flag);
      break;
    case 4:
      hipLaunchKernelGGL((tile_copy_kernel<4, 4>), grid, dim3(256), 0, stream, s, d, g,
                         (uint32_t)row_bytes, fu, fw, fh, flag);
      break;
    default:
      hipLaunchKernelGGL((tile_copy_kernel<2, 4>), grid, dim3(256), 0, stream, s, d, g,
                         (uint32_t)row_bytes, fu, fw, fh, flag);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tile-pair enumeration.  Count of key tiles seen by any query tile of a head:
// prod_d w'_d.  Transposed: key tile k is seen by the query tiles of an
// interval per dimension (window_transpose), so its count is a product too.
// ---------------------------------------------------------------------------
STA_HD int64_t transposed_count(int k0, int k1, int k2, const uint16_t* wp, const Geometry& g) {
  int lo, hi;
  int64_t c = 1;
  window_transpose(k0, wp[0], g.n0, &lo, &hi);
  c *= (hi - lo + 1);
  window_transpose(k1, wp[1], g.n1, &lo, &hi);
  c *= (hi - lo + 1);
  window_transpose(k2, wp[2], g.n2, &lo, &hi);
  c *= (hi - lo + 1);
  return c;
}

// Writes the pairs of tile `a` of head `hh` (a = query tile in the forward view,
// key tile in the transposed view) starting at out[pos].
STA_HD void emit_tile_pairs(int32_t* out, int64_t pos, int a, const uint16_t* wp, const Geometry& g,
                            int transpose) {
  const int a2 = a % g.n2, a1 = (a / g.n2) % g.n1, a0 = a / (g.n2 * g.n1);
  if (!transpose) {
    const int s0 = window_start(a0, wp[0], g.n0), s1 = window_start(a1, wp[1], g.n1),
              s2 = window_start(a2, wp[2], g.n2);
    for (int i0 = 0; i0 < wp[0]; ++i0)
      for (int i1 = 0; i1 < wp[1]; ++i1)
        for (int i2 = 0; i2 < wp[2]; ++i2) {
          out[2 * pos] = a;
          out[2 * pos + 1] = ((s0 + i0) * g.n1 + (s1 + i1)) * g.n2 + (s2 + i2);
          ++pos;
        }
  } else {
    int l0, h0, l1, h1, l2, h2;
    window_transpose(a0, wp[0], g.n0, &l0, &h0);
    window_transpose(a1, wp[1], g.n1, &l1, &h1);
    window_transpose(a2, wp[2], g.n2, &l2, &h2);
    for (int q0 = l0; q0 <= h0; ++q0)
      for (int q1 = l1; q1 <= h1; ++q1)
        for (int q2 = l2; q2 <= h2; ++q2) {
          out[2 * pos] = (q0 * g.n1 + q1) * g.n2 + q2;
          out[2 * pos + 1] = a;
          ++pos;
        }
  }
}

// Start of tile a's pairs inside its head's list.
STA_HD int64_t tile_pair_offset(int a, const uint16_t* wp, const Geometry& g, int transpose) {
  if (!transpose) return (int64_t)a * wp[0] * wp[1] * wp[2];
  int64_t pos = 0;
  for (int k = 0; k < a; ++k)
    pos += transposed_count(k / (g.n2 * g.n1), (k / g.n2) % g.n1, k % g.n2, wp, g);
  return pos;
}

__global__ __launch_bounds__(256) void tile_pairs_kernel(int32_t* out, Geometry g, HeadTable ht,
                                                         int Hh, int transpose) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id >= Hh * g.ntiles) return;
  const int hh = id / g.ntiles, a = id % g.ntiles;
  int64_t pos = 0;
  for (int j = 0; j < hh; ++j) pos += (int64_t)g.ntiles * ht.wp[j][0] * ht.wp[j][1] * ht.wp[j][2];
  pos += tile_pair_offset(a, ht.wp[hh], g, transpose);
  emit_tile_pairs(out, pos, a, ht.wp[hh], g, transpose);
}

hipError_t launch_tile_pairs(int32_t* out, const Geometry& g, const HeadTable& ht, int Hh,
                             int transpose, hipStream_t stream) {
  const int n = Hh * g.ntiles;
  hipLaunchKernelGGL(tile_pairs_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, out, g, ht,
                     Hh, transpose);
  return hipGetLastError();
}

void host_tile_pairs(int32_t* out, const Geometry& g, const HeadTable& ht, int Hh, int transpose) {
  int64_t pos = 0;
  for (int hh = 0; hh < Hh; ++hh)
    for (int a = 0; a < g.ntiles; ++a) {
      emit_tile_pairs(out, pos, a, ht.wp[hh], g, transpose);
      pos += transpose ? transposed_count(a / (g.n2 * g.n1), (a / g.n2) % g.n1, a % g.n2,
                                          ht.wp[hh], g)
                       : (int64_t)ht.wp[hh][0] * ht.wp[hh][1] * ht.wp[hh][2];
    }
}

}  // namespace sta
