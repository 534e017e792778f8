// STA forward, bf16 in/out, fp32 accumulation, on gfx950 MFMA.
//
// "Sliding Tile Attention" (arXiv 2502.04507 summary page, abstract and method
// details): each query tile attends densely to the key tiles of its window, so
// every (query block, key block) product below is a full dense contraction.
// The only mask is the padding one of latents that are not a whole number of
// tiles (OpenReview rebuttal, answer on input resolution), applied to the key
// blocks of partial tiles only.
//
// Work decomposition
//   One workgroup = NW waves = NW*QT*32 query rows of one query tile of one
//   (batch, head).  Each wave keeps its QT*32 query rows resident in registers
//   for the whole key walk.  The key tiles of the window are walked in KB-key
//   blocks through a ring of LDS slots filled by 16-byte global->LDS DMA.
// Instances: tile-major tensors (sta_forward, sta_dense_forward), raster-order
//   tensors with the reorder folded into the loads and stores
//   (sta_forward_raster), and the normaliser (log-sum-exp) alone, K only and
//   no P V (sta_window_mass).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16)
//   S^T = K Q^T     A = K rows (LDS), B = Q^T (registers).  Lane l of the
//                   accumulator holds query l % 32 against 16 keys, so the row
//                   statistics are per-lane scalars plus one exchange with lane
//                   l ^ 32.
//   O^T += V^T P^T  A = V^T read from the row-major V tile with the gfx950
//                   transposed LDS read, B = P^T taken straight from the S^T
//                   accumulator (converted to bf16).  Lane l keeps query l % 32,
//                   so the output rescale and the final 1/l are per-lane scalars.
//   Inside each 16-key MFMA step the key order follows the accumulator layout:
//   slot 8g + 4u + j holds key 8u + 4g + j; the V^T reads use the same order.
//
// Softmax: scores are scaled by scale*log2(e) inside one FMA and exponentiated
// with exp2.  The running maximum is only raised (and O, l rescaled) when a
// block's maximum exceeds it by more than 8 (a factor 256): probabilities stay
// below 256, and O and l are always scaled by the same factor, so the result is
// exact in real arithmetic.
#include "kernels.h"
#include "mfma_common.h"

namespace sta {

namespace {

constexpr float kRescaleThreshold = 8.0f;
// Copy segments per tile the raster instance tabulates (L / rows-per-segment).
constexpr int kMaxRasterSegs = 1024;

template <int D, int QT, int NW>
struct FwdCfg {
  static constexpr int KB = 32;              // keys per LDS stage (one MFMA sub-tile)
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWS = NW * QT * 32;  // query rows per workgroup
  static constexpr int KS = D / 16;          // MFMA k-steps of K Q^T
  static constexpr int DT = D / 32;          // 32-wide d tiles of O^T
  static constexpr int TILE_BYTES = KB * D * 2;
};

// S^T = K Q^T for one 32-key stage.
template <int D, int QT>
__device__ __forceinline__ void qk_stage(const bf16x8 (&kf)[D / 16], const bf16x8 (&qf)[QT][D / 16],
                                         f32x16 (&sacc)[QT]) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) sacc[qt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sacc[qt] = mfma32(kf[ks], qf[qt][ks], sacc[qt]);
}

// Maximum of a block's 16 scores as a balanced tree (depth 4).  The IEEE
// maximum (NaN-propagating) needs no operand canonicalisation, which fmaxf
// (maxNum) inserts for every operand coming straight from an MFMA; the
// scores are finite, so both give the same value.
__device__ __forceinline__ float vmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax2(vmax2(a, b), c); }
__device__ __forceinline__ float block_max16(const f32x16& s) {
  const float m0 = vmax3(s[0], s[1], s[2]), m1 = vmax3(s[3], s[4], s[5]), m2 = vmax3(s[6], s[7], s[8]);
  const float m3 = vmax3(s[9], s[10], s[11]), m4 = vmax3(s[12], s[13], s[14]);
  return vmax2(vmax3(m0, m1, m2), vmax3(m3, m4, s[15]));
}
// The same across the two lanes l and l ^ 32 that hold one query's scores.
__device__ __forceinline__ float xmax32_raw(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax2(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

// Online softmax of one stage (lazy rescale), producing the bf16 P^T operand.
// mlim = mrun + the rescale threshold, kept beside mrun so that a stage
// compares without an add.
template <int D, int QT>
__device__ __forceinline__ void softmax_stage(const f32x16 (&sacc)[QT], bf16x8 (&pf)[QT][2],
                                              f32x16 (&oacc)[QT][D / 32], float (&mrun)[QT],
                                              float (&mlim)[QT], float (&lrun)[QT], float c_log2) {
  bool need = false;
  float mblk[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mblk[qt] = xmax32_raw(block_max16(sacc[qt])) * c_log2;
    need |= mblk[qt] > mlim[qt];
  }
  if (__any(need)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mn = vmax2(mrun[qt], mblk[qt]);  // finite block maxima: no NaN to order
      const float alpha = __builtin_amdgcn_exp2f(mrun[qt] - mn);
      mrun[qt] = mn;
      mlim[qt] = mn + kRescaleThreshold;
      lrun[qt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[qt][dt][e] *= alpha;
    }
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float mneg = -mrun[qt];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[qt][s][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[qt][8 * s + e], c_log2, mneg));
    // Row sum of the bf16 probabilities (the values P V uses), two per dot2,
    // accumulated straight into the running sum.
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lrun[qt] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[qt][s][2 * e], pf[qt][s][2 * e + 1]}, one,
                                                   lrun[qt], false);
  }
}

// Softmax normaliser only (no P V), for the window mass: running maximum and
// fp32 row sums of the exponentials, with the same lazy rescale.  The current
// key tile's sum collects in ltile; at the tile's last block it joins the full
// sum and the sums of the candidate windows that hold the tile (member bit c).
template <int QT>
__device__ __forceinline__ void mass_stage(const f32x16 (&sacc)[QT], float (&mrun)[QT],
                                           float (&lfull)[QT], float (&ltile)[QT],
                                           float (&lc)[QT][kMaxCandidates], int ncand,
                                           bool tile_done, uint32_t member, float c_log2) {
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float mblk = xmax32_raw(block_max16(sacc[qt])) * c_log2;
    if (mblk > mrun[qt] + kRescaleThreshold) {
      const float alpha = __builtin_amdgcn_exp2f(mrun[qt] - mblk);
      lfull[qt] *= alpha;
      ltile[qt] *= alpha;
#pragma unroll
      for (int c = 0; c < kMaxCandidates; ++c) lc[qt][c] *= alpha;
      mrun[qt] = mblk;
    }
    const float mneg = -mrun[qt];
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(sacc[qt][e], c_log2, mneg));
#pragma unroll
    for (int w = 8; w > 0; w >>= 1)  // pairwise tree: depth 4 instead of a 16-add chain
#pragma unroll
      for (int e = 0; e < w; ++e) pe[e] += pe[e + w];
    ltile[qt] += pe[0];
    if (tile_done) {
      lfull[qt] += ltile[qt];
#pragma unroll
      for (int c = 0; c < kMaxCandidates; ++c)
        if (c < ncand && ((member >> c) & 1u)) lc[qt][c] += ltile[qt];
      ltile[qt] = 0.f;
    }
  }
}

// O^T += V^T P^T for one stage.
template <int D, int QT>
__device__ __forceinline__ void pv_stage(const bf16x8 (&vf)[D / 32][2], const bf16x8 (&pf)[QT][2],
                                         f32x16 (&oacc)[QT][D / 32]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) oacc[qt][dt] = mfma32(vf[dt][s], pf[qt][s], oacc[qt][dt]);
}

// Raster row (inside its sequence) of intra-tile position r of tile
// (a0, a1, a2): the tile-major -> raster map of the reorder, for one row.
__device__ __forceinline__ uint32_t raster_row(int a0, int a1, int a2, uint32_t r,
                                               const Geometry& g) {
  const uint32_t i0 = fdiv(r, g.fhw), rem = r - i0 * (uint32_t)(g.h * g.w);
  const uint32_t i1 = fdiv(rem, g.fw), i2 = rem - i1 * (uint32_t)g.w;
  return ((uint32_t)(a0 * g.t) + i0) * (uint32_t)g.H * (uint32_t)g.W +
         ((uint32_t)(a1 * g.h) + i1) * (uint32_t)g.W + (uint32_t)(a2 * g.w) + i2;
}

// MASS: the window mass (v and o unused): K blocks only, no P V; the head
// table holds the full window and ma the candidate windows (see MassArgs).
// RASTER: q, k, v, o and lse are in raster order (a latent whose tile width
// is a multiple of a copy segment's rows): the reorder and unreorder happen in
// the kernel's own loads and stores.  With padding (PADM != 0) the raster
// tensors hold only the real tokens.
template <int D, int QT, int NW, int OCC, bool MASS, bool RASTER, int PADM>
__global__ __launch_bounds__(64 * NW, OCC) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, Geometry g,
    HeadTable ht, MassArgs ma, int B, int Hh, float c_log2, int blocks_per_tile, int total,
    int group_items) {
  using C = FwdCfg<D, QT, NW>;
  constexpr int KB = C::KB;
  // A ring of four stages, each buffer its own object so the compiler can
  // tell the DMA targets from the buffers being read.
  __shared__ __attribute__((aligned(1024))) char kl0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vl0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kl1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vl1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kl2[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vl2[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kl3[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vl3[C::TILE_BYTES];

  // Work item.  Workgroups are dealt round-robin to the 8 XCDs (XCD x runs
  // every 8th blockIdx).  Items are ordered (head slot, batch, query tile,
  // sub-block); consecutive groups of group_items items (one or a few whole
  // (head, batch) sequences, a multiple of 8) are split into 8 contiguous
  // chunks, chunk x going to XCD x.  So all XCDs work on the same few heads at
  // a time (their K/V stays in the shared last-level cache) and each XCD walks
  // neighbouring query tiles (its L2 sees overlapping windows).  group_items ==
  // 0 (no such grouping exists) falls back to one contiguous range per XCD.
  const uint32_t bid = blockIdx.x;
  const uint32_t xcd = bid & 7u, local = bid >> 3;
  uint32_t item;
  if (group_items > 0) {
    const uint32_t per_x = (uint32_t)group_items >> 3;
    item = (local / per_x) * (uint32_t)group_items + xcd * per_x + local % per_x;
  } else {
    const uint32_t per = (uint32_t)total >> 3, rem = (uint32_t)total & 7u;
    item = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  }
  const int sub = item % blocks_per_tile;
  item /= blocks_per_tile;
  const int qtile = item % g.ntiles;
  item /= g.ntiles;
  const int b = item % B;
  const int head = ht.order[item / B];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 5, c32 = lane & 31;

  // Rows per (batch, head) sequence: the padded tile-major length, or, for
  // a raster-order tensor (real tokens only), T*H*W.
  const size_t seq = ((size_t)b * Hh + head) * (size_t)(RASTER ? g.Sr : g.S);
  const uint16_t* kb = k + seq * D;
  const uint16_t* vb = v + seq * D;

  // Window of this query tile.
  const int a2 = qtile % g.n2, a1 = (qtile / g.n2) % g.n1, a0 = qtile / (g.n2 * g.n1);

  // Q^T fragments (B operand): lane holds 8 consecutive d of its query row.
  // qrow[qt]: the lane's query row inside the sequence (tile-major, or its
  // raster position).
  // Padded latents: the real query rows of a partial tile are taken
  // compacted, as the keys below: workgroup sub of the tile takes compacted
  // rows [sub * ROWS, (sub + 1) * ROWS), so the tile needs ceil(real / ROWS)
  // workgroups and the rest find no real row.  A lane past the real count
  // has no query: it loads zeros and writes nothing for it.
  const int qrow0 = qtile * g.L + sub * C::ROWS + wave * QT * 32;
  int qn = g.L;  // real query rows of the tile
  int qe1 = g.h, qe2 = g.w;
  if constexpr (PADM != 0) {
    qe1 = tile_ext(a1, g.h, g.H);
    qe2 = tile_ext(a2, g.w, g.W);
    qn = tile_ext(a0, g.t, g.T) * qe1 * qe2;
  }
  uint32_t qrow[QT];
  bool qreal[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int ci = qrow0 - qtile * g.L + qt * 32 + c32;  // row inside the tile (compacted if padded)
    uint32_t r = (uint32_t)ci;
    qreal[qt] = PADM == 0 || ci < qn;
    if (PADM != 0 && qn < g.L) {
      const TilePos tp = split_compact((uint32_t)ci, qe1, qe2, __builtin_amdgcn_rcpf((float)qe1),
                                       __builtin_amdgcn_rcpf((float)qe2));
      r = (tp.t * (uint32_t)g.h + tp.h) * (uint32_t)g.w + tp.w;
    }
    qrow[qt] = !qreal[qt] ? 0u : RASTER ? raster_row(a0, a1, a2, r, g) : (uint32_t)(qtile * g.L) + r;
  }
  bf16x8 qf[QT][C::KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[qt][ks] = qreal[qt] ? as_bf16x8(*(const u32x4*)(q + (seq + qrow[qt]) * D + ks * 16 + grp * 8))
                             : bf16x8{};
  const int w0 = ht.wp[head][0], w1 = ht.wp[head][1], w2 = ht.wp[head][2];
  const int s0 = window_start(a0, w0, g.n0), s1 = window_start(a1, w1, g.n1),
            s2 = window_start(a2, w2, g.n2);
  const int bpt = g.L / KB;
  // Padded latents (PADM 1): the real keys of a partial key tile are walked
  // compacted, in the tile's own (t, h, w) order with the padding positions
  // left out, so the tile takes ceil(real keys / 32) blocks and only the last
  // of them can hold padding, at its end.  Whole tiles are walked as they
  // are (L / 32 blocks).  Only the last tile along an axis is partial, so the
  // window's block count is a sum over the 8 classes (last along t, h, w or
  // not) of the class's tile count times its blocks.
  auto tile_blocks = [&](int e0, int e1, int e2) -> int { return (e0 * e1 * e2 + KB - 1) / KB; };
  int nblk = w0 * w1 * w2 * bpt;
  if constexpr (PADM != 0) {
    const int x0 = tile_ext(g.n0 - 1, g.t, g.T), x1 = tile_ext(g.n1 - 1, g.h, g.H),
              x2 = tile_ext(g.n2 - 1, g.w, g.W);
    const int l0 = s0 + w0 == g.n0, l1 = s1 + w1 == g.n1, l2 = s2 + w2 == g.n2;
    nblk = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int c0 = c & 1, c1 = (c >> 1) & 1, c2 = c >> 2;
      const int cnt = (c0 ? l0 : w0 - l0) * (c1 ? l1 : w1 - l1) * (c2 ? l2 : w2 - l2);
      nblk += cnt * tile_blocks(c0 ? x0 : g.t, c1 ? x1 : g.h, c2 ? x2 : g.w);
    }
    if (sub * C::ROWS >= qn) nblk = 0;  // no real query row here: straight to the epilogue
  }

  // Mass instance: the start of every candidate window of this query tile
  // (fixed for the whole walk).
  int cs[MASS ? kMaxCandidates : 1][3];
  if constexpr (MASS) {
#pragma unroll
    for (int c = 0; c < kMaxCandidates; ++c) {
      const bool use = c < ma.ncand;
      cs[c][0] = use ? window_start(a0, ma.w[c][0], g.n0) : 0;
      cs[c][1] = use ? window_start(a1, ma.w[c][1], g.n1) : 0;
      cs[c][2] = use ? window_start(a2, ma.w[c][2], g.n2) : 0;
    }
  }

  int i0 = 0, i1 = 0, i2 = 0, jb = 0;  // key-block walk, incremented
  int kbt = bpt;                        // blocks of the walk's key tile
  // The walk's key tile, worked out when the walk reaches it, not per block:
  // its first row (korg: tile-major, or the raster row of its origin); with
  // padding its real extent per axis, its real key count (knreal) and, for a
  // partial tile, the reciprocals of its real extent along h and w (the
  // compacted key index is split into (t, h, w) with them); in the mass
  // instance the candidate windows that hold it (kmember, one bit each).
  uint32_t korg = 0;
  int ke1 = g.h, ke2 = g.w, knreal = g.L;
  bool kpart = false;
  float kinv1 = 1.0f, kinv2 = 1.0f;
  uint32_t kmember = 0;
  auto enter_tile = [&]() __attribute__((always_inline)) {
    const int k0 = s0 + i0, k1 = s1 + i1, k2 = s2 + i2;
    if constexpr (!RASTER)
      korg = (uint32_t)(((k0 * g.n1 + k1) * g.n2 + k2) * g.L);
    else
      korg = ((uint32_t)(k0 * g.t) * (uint32_t)g.H + (uint32_t)(k1 * g.h)) * (uint32_t)g.W +
             (uint32_t)(k2 * g.w);
    if constexpr (PADM != 0) {
      const int e0 = tile_ext(k0, g.t, g.T);
      ke1 = tile_ext(k1, g.h, g.H);
      ke2 = tile_ext(k2, g.w, g.W);
      knreal = e0 * ke1 * ke2;
      kpart = knreal < g.L;
      kbt = tile_blocks(e0, ke1, ke2);
      if (kpart) {  // (scalar registers: the same in every lane)
        kinv1 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_amdgcn_rcpf((float)ke1))));
        kinv2 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_amdgcn_rcpf((float)ke2))));
      }
    }
    if constexpr (MASS) {
      kmember = 0;
#pragma unroll
      for (int c = 0; c < kMaxCandidates; ++c) {
        if (c < ma.ncand) {
          const bool in = (unsigned)(k0 - cs[c][0]) < (unsigned)ma.w[c][0] &&
                          (unsigned)(k1 - cs[c][1]) < (unsigned)ma.w[c][1] &&
                          (unsigned)(k2 - cs[c][2]) < (unsigned)ma.w[c][2];
          kmember |= (in ? 1u : 0u) << c;
        }
      }
    }
  };
  enter_tile();
  auto next_block = [&]() __attribute__((always_inline)) {
    if (++jb == kbt) {
      jb = 0;
      if (++i2 == w2) {
        i2 = 0;
        if (++i1 == w1) {
          i1 = 0;
          ++i0;
        }
      }
      enter_tile();
    }
  };
  // Raster instance: the intra-tile part of the raster row of each copy
  // segment's first row (the same for every whole key tile), tabulated once;
  // a segment's raster row is then its key tile's origin plus the entry.
  __shared__ uint32_t seg_intra[RASTER ? kMaxRasterSegs : 1];
  if constexpr (RASTER) {
    constexpr int RPS = KvDma<D, KB, NW>::RPS;
    for (int i = tid; i < g.L / RPS; i += C::THREADS) {
      const uint32_t r = (uint32_t)(i * RPS);
      const uint32_t t0 = fdiv(r, g.fhw), rem = r - t0 * (uint32_t)(g.h * g.w);
      const uint32_t t1 = fdiv(rem, g.fw), t2 = rem - t1 * (uint32_t)g.w;
      seg_intra[i] = (t0 * (uint32_t)g.H + t1) * (uint32_t)g.W + t2;
    }
    __syncthreads();
  }
  using Cp = KvDma<D, KB, NW>;
  const Cp copier(__builtin_amdgcn_readfirstlane(wave), lane);
  // What the stage computing a block needs beyond its keys, worked out when
  // the block's copy is issued and kept beside its ring slot (the loops are
  // unrolled by the slot count, so each slot's copy is a fixed register):
  //   nvalid: padded latents, the real keys of a block that ends a partial
  //           key tile with padding (1..31); 0 for a block of real keys only;
  //   mass:   bits 0-7 the candidate windows holding the block's key tile,
  //           bit 31 set when the block is its tile's last.
  struct BlockInfo {
    uint32_t nvalid;
    uint32_t mass;
  };
  // A partial key tile's block: the lane's key of each of its copy segments
  // is compacted key c = jb * 32 + row of the tile.
  auto issue = [&](char* kl, char* vl, BlockInfo& bi) __attribute__((always_inline)) {
    if constexpr (PADM != 0) bi.nvalid = jb == kbt - 1 ? (uint32_t)(knreal - jb * KB) & (KB - 1) : 0u;
    if constexpr (MASS) bi.mass = kmember | (jb == kbt - 1 ? 0x80000000u : 0u);
    const uint32_t org = korg;
    if (PADM != 0 && kpart) {
      const uint32_t sa = RASTER ? (uint32_t)(g.H * g.W) : (uint32_t)(g.h * g.w);
      const uint32_t sb = RASTER ? (uint32_t)g.W : (uint32_t)g.w;
      uint32_t rel[Cp::PT];
      bool real[Cp::PT];
#pragma unroll
      for (int e = 0; e < Cp::PT; ++e) {
        const uint32_t c = (uint32_t)(jb * KB) + copier.row_in_block(e, lane);
        const TilePos tp = split_compact(c, ke1, ke2, kinv1, kinv2);
        real[e] = c < (uint32_t)knreal;
        rel[e] = tp.t * sa + tp.h * sb + tp.w;
      }
      next_block();
      if constexpr (MASS)
        copier.issue_k_gather(kb, org, rel, real, kl);
      else
        copier.issue_rows_gather(kb, vb, org, rel, real, kl, vl);
    } else if constexpr (RASTER) {
      // raster rows of this block's segments (scalar: the same in every lane),
      // one scalar base per tensor and a 32-bit lane offset per segment
      uint32_t offs[Cp::PT];
#pragma unroll
      for (int e = 0; e < Cp::PT; ++e)
        offs[e] = __builtin_amdgcn_readfirstlane(seg_intra[jb * (KB / Cp::RPS) + copier.wave_u + e * NW]);
      next_block();
      copier.issue_rows_origin(kb, vb, org, offs, kl, vl);
    } else {
      const size_t row0 = (size_t)org + (size_t)(jb * KB);
      next_block();
      if constexpr (MASS)
        copier.issue_k(kb, row0, kl);
      else
        copier.issue(kb, vb, row0, kl, vl);
    }
  };

  // Padding mask: element e of lane l in the S^T accumulator holds key
  // 8 (e / 4) + 4 (l / 32) + e % 4 of the block, so with compacted keys a
  // stage whose block ends a partial tile sets the scores of keys at or past
  // its real count to -inf (a select, so whatever the staged padding row
  // holds is masked exactly).
  auto mask_keys = [&](f32x16 (&sacc)[QT], const BlockInfo& bi) {
    if constexpr (PADM != 0) {
      if (bi.nvalid != 0u) {  // uniform
        // 4 (l / 32) worked out here, not held in a register across the loop
        uint32_t l = (uint32_t)lane;
        asm volatile("" : "+v"(l));
        const int nv = (int)bi.nvalid - (int)((l >> 5) << 2);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool real = 8 * (e >> 2) + (e & 3) < nv;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) sacc[qt][e] = real ? sacc[qt][e] : -INFINITY;
        }
      }
    }
  };

  f32x16 oacc[QT][C::DT];
  float mrun[QT], mlim[QT], lrun[QT];
  float ltile[QT], lcand[QT][kMaxCandidates];  // mass instance only
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[qt][dt] = f32x16{};
    mrun[qt] = -INFINITY;
    mlim[qt] = -INFINITY;
    lrun[qt] = 0.f;
    ltile[qt] = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxCandidates; ++c) lcand[qt][c] = 0.f;
  }

  // Pipeline over 32-key stages; stage j sits in LDS slot j % SLOTS.  Four
  // slots for 4-wave workgroups; two for smaller workgroups, whose 64 KB
  // four-slot ring would leave room for only two of them per CU (one wave per
  // SIMD), while at 32 KB four fit and each SIMD runs two waves.  In stage j:
  // Q K^T and softmax of j (its K fragments were read in stage j - 1); wait
  // for the copy of stage j + 1 (with four slots the copy of j + 2 stays in
  // flight); barrier; read the K and V^T fragments of j + 1; start the copy of
  // stage j + AHEAD into the slot that is free: (j + 3) % 4, last read in
  // stage j - 2, or with two slots j % 2, read in stage j - 1 (each wave waits
  // for its own LDS reads before the barrier, so none is still in flight);
  // then P V of j, overlapping the reads.
  constexpr int SLOTS = NW >= 4 ? 4 : 2;
  constexpr int AHEAD = SLOTS == 4 ? 3 : 2;
  constexpr int PER = MASS ? KvDma<D, KB, NW>::PT : KvDma<D, KB, NW>::PER;
  BlockInfo bi0{}, bi1{}, bi2{}, bi3{};  // ring slots 0..3
  if (nblk > 0) issue(kl0, vl0, bi0);
  if (nblk > 1) issue(kl1, vl1, bi1);
  if constexpr (SLOTS == 4) {
    if (nblk > 2) issue(kl2, vl2, bi2);
    if (nblk > 2) wait_dma_upto<2 * PER>();
    else wait_dma();
  } else {
    if (nblk > 1) wait_dma_upto<PER>();
    else wait_dma();
  }
  barrier_lds();
  auto wait_next = [&](int j) {
    if constexpr (SLOTS == 4) {
      if (j + 2 < nblk) wait_dma_upto<PER>();
      else wait_dma();
    } else {
      wait_dma();
      wait_lds();
    }
  };
  // Each stage reads all its operands of the next stage before it starts a
  // copy (reads behind the wave's own copy were measured slower).
  bf16x8 kf[C::KS], vfa[C::DT][2], vfb[C::DT][2];
  read_rows<D>(kl0, kf, grp, c32);
  if constexpr (!MASS) read_cols<D>(vl0, vfa, lane);

  // bi_cur describes stage j's block, bi_far receives the block copied into
  // the slot being refilled (the same slot with two slots: bi_cur is read
  // before the copy is issued).
  auto stage = [&](int j, bf16x8 (&vf)[C::DT][2], bf16x8 (&vf_nxt)[C::DT][2], const char* kl_nxt,
                   const char* vl_nxt, char* kl_far, char* vl_far, const BlockInfo& bi_cur,
                   BlockInfo& bi_far) {
    f32x16 sacc[QT];
    qk_stage<D, QT>(kf, qf, sacc);
    mask_keys(sacc, bi_cur);
    if constexpr (MASS) {
      const bool tile_done = (bi_cur.mass >> 31) != 0u;
      const uint32_t member = bi_cur.mass & 0xffu;
      mass_stage<QT>(sacc, mrun, lrun, ltile, lcand, ma.ncand, tile_done, member, c_log2);
      if (j + 1 < nblk) {
        wait_next(j);
        barrier_lds();
        read_rows<D>(kl_nxt, kf, grp, c32);
        asm volatile("" ::: "memory");
        if (j + AHEAD < nblk) issue(kl_far, vl_far, bi_far);
      }
      return;
    }
    bf16x8 pf[QT][2];
    // Raised wave priority during the vector work: when the two waves of a
    // SIMD compete for issue, the one in its softmax goes first and the
    // other's matrix instructions fill the gaps (measured +2%).
    __builtin_amdgcn_s_setprio(2);
    softmax_stage<D, QT>(sacc, pf, oacc, mrun, mlim, lrun, c_log2);
    __builtin_amdgcn_s_setprio(0);
    if (j + 1 < nblk) {
      wait_next(j);
      barrier_lds();
      read_rows<D>(kl_nxt, kf, grp, c32);
      read_cols<D>(vl_nxt, vf_nxt, lane);
      asm volatile("" ::: "memory");
      if (j + AHEAD < nblk) issue(kl_far, vl_far, bi_far);
    }
    pv_stage<D, QT>(vf, pf, oacc);
  };
  // A wave whose query rows are all padding (a padded latent) computes
  // nothing: it waits, joins every barrier and issues its share of the
  // copies like the others, and its outputs are the padding rows' zeros.
  bool any_real = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) any_real |= qreal[qt];
  if (PADM != 0 && __ballot(any_real) == 0) {
    BlockInfo unused{};
    auto idle = [&](int j, char* kl_far, char* vl_far) {
      if (j + 1 < nblk) {
        wait_next(j);
        barrier_lds();
        if (j + AHEAD < nblk) issue(kl_far, vl_far, unused);
      }
    };
    if constexpr (SLOTS == 4) {
      for (int j = 0; j < nblk; j += 4) {
        idle(j, kl3, vl3);
        idle(j + 1, kl0, vl0);
        idle(j + 2, kl1, vl1);
        idle(j + 3, kl2, vl2);
      }
    } else {
      for (int j = 0; j < nblk; j += 2) {
        idle(j, kl0, vl0);
        idle(j + 1, kl1, vl1);
      }
    }
  } else if constexpr (SLOTS == 4) {
    // stage j reads slot (j + 1) % 4 and refills slot (j + 3) % 4
    for (int j = 0; j < nblk; j += 4) {
      stage(j, vfa, vfb, kl1, vl1, kl3, vl3, bi0, bi3);
      if (j + 1 >= nblk) break;
      stage(j + 1, vfb, vfa, kl2, vl2, kl0, vl0, bi1, bi0);
      if (j + 2 >= nblk) break;
      stage(j + 2, vfa, vfb, kl3, vl3, kl1, vl1, bi2, bi1);
      if (j + 3 >= nblk) break;
      stage(j + 3, vfb, vfa, kl0, vl0, kl2, vl2, bi3, bi2);
    }
  } else {
    // stage j reads slot (j + 1) % 2 and refills slot j % 2 (read by every
    // wave one stage earlier)
    for (int j = 0; j < nblk; j += 2) {
      stage(j, vfa, vfb, kl1, vl1, kl0, vl0, bi0, bi0);
      if (j + 1 >= nblk) break;
      stage(j + 1, vfb, vfa, kl0, vl0, kl1, vl1, bi1, bi1);
    }
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 on the lane's query row.
  // Padded tile-major tensors: each lane also writes zeros (O and LSE) to
  // the row at its uncompacted position when that position is padding, so
  // every padding row of the tile is zeroed once and every real row is
  // written once, by the lane that took it.
  // Mass instance: row mass l_c / l per candidate, summed over the wave's 32
  // rows into one partial per (candidate, sequence, 32-row block).
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = xsum32(lrun[qt]);
    const bool real = qreal[qt];
    const float inv = real ? 1.0f / lt : 0.0f;
    const size_t row = seq + qrow[qt];
    if constexpr (PADM != 0 && !RASTER) {
      const int pos = qrow0 - qtile * g.L + qt * 32 + c32;  // uncompacted position in the tile
      if (!token_real(a0, a1, a2, pos, g)) {
        const size_t prow = seq + (size_t)(qtile * g.L + pos);
        if constexpr (!MASS) {
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) *(bf16x4*)(o + prow * D + dt * 32 + 8 * i + 4 * grp) = bf16x4{};
        } else if (ma.lse_last != nullptr && grp == 0) {
          ma.lse_last[prow] = 0.0f;
        }
        if (lse != nullptr && grp == 0) lse[prow] = 0.0f;
      }
    }
    if constexpr (!MASS) {
      if (!real) continue;  // no query row
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[qt][dt][4 * i + j] * inv);
          *(bf16x4*)(o + row * D + dt * 32 + 8 * i + 4 * grp) = w;
        }
    } else {
      const size_t bh = (size_t)b * Hh + head;
      const size_t nblk32 = (size_t)g.S / 32;
      const size_t blk = (size_t)(qrow0 + qt * 32) / 32;
#pragma unroll
      for (int c = 0; c < kMaxCandidates; ++c) {
        if (c < ma.ncand) {
          const float lcs = xsum32(lcand[qt][c]);
          float r = real ? lcs * inv : 0.0f;  // a select: 0 past the real rows
          // sum over the 32 rows (lanes 0..31; lanes 32..63 hold the same rows)
#pragma unroll
          for (int off = 16; off > 0; off >>= 1) r += __shfl_xor(r, off, 32);
          if (lane == 0) ma.partial[((size_t)c * B * Hh + bh) * nblk32 + blk] = r;
          if (c == ma.ncand - 1 && ma.lse_last != nullptr && grp == 0 && real)
            ma.lse_last[row] = (mrun[qt] + log2f(lcs)) * kLn2;
        }
      }
      if (!real) continue;
    }
    if (lse != nullptr && grp == 0) lse[row] = (mrun[qt] + log2f(lt)) * kLn2;
  }
}

// Items per XCD-split group: the smallest number of whole (head, batch)
// sequences whose item count is a multiple of 8 and divides the total; 0 if
// there is none.
inline int xcd_group_items(int seqs, int items_per_seq) {
  for (int gsz = 1; gsz <= 8; ++gsz)
    if ((gsz * items_per_seq) % 8 == 0 && seqs % gsz == 0) return gsz * items_per_seq;
  return 0;
}

template <int D, int QT, int NW, int OCC, bool MASS = false, bool RASTER = false>
hipError_t launch_cfg(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                      float* lse, const Geometry& g, const HeadTable& ht, int B, int Hh,
                      float scale, hipStream_t st, const MassArgs& ma = MassArgs{}) {
  using C = FwdCfg<D, QT, NW>;
  const int bpt = g.L / C::ROWS;
  const int total = B * Hh * g.ntiles * bpt;
  const int group = xcd_group_items(B * Hh, g.ntiles * bpt);
  // Padded latents get an instance of their own (compacted keys of partial
  // tiles, the key mask, the zeroed or skipped padding rows).
  if (g.padded) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, NW, OCC, MASS, RASTER, 1>), dim3((uint32_t)total),
                       dim3(C::THREADS), 0, st, q, k, v, o, lse, g, ht, ma, B, Hh, scale * kLog2e,
                       bpt, total, group);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, NW, OCC, MASS, RASTER, 0>), dim3((uint32_t)total),
                     dim3(C::THREADS), 0, st, q, k, v, o, lse, g, ht, ma, B, Hh, scale * kLog2e,
                     bpt, total, group);
  return hipGetLastError();
}

}  // namespace

// A padded latent's compacted key index (below L) is split with fp32
// reciprocals, exact for indices below 2^21.
bool fwd_bf16_supported(int D, const Geometry& g) {
  return (D == 64 || D == 128) && g.L % 32 == 0 && (!g.padded || g.L <= (1 << 20));
}

template <bool RASTER>
hipError_t launch_fwd_order(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                            float* lse, const Geometry& g, const HeadTable& ht, int B, int Hh,
                            int D, float scale, hipStream_t st) {
  const int L = g.L;
  if (D == 128) {
    if (L % 128 == 0)
      return launch_cfg<128, 1, 4, 2, false, RASTER>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    if (L % 64 == 0)
      return launch_cfg<128, 1, 2, 2, false, RASTER>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    return launch_cfg<128, 1, 1, 1, false, RASTER>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
  }
  if (D == 64) {
    if (L % 128 == 0)
      return launch_cfg<64, 1, 4, 2, false, RASTER>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    if (L % 64 == 0)
      return launch_cfg<64, 1, 2, 2, false, RASTER>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    return launch_cfg<64, 1, 1, 1, false, RASTER>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, const Geometry& g, const HeadTable& ht, int B, int Hh,
                           int D, float scale, hipStream_t st) {
  return launch_fwd_order<false>(q, k, v, o, lse, g, ht, B, Hh, D, scale, st);
}

bool fwd_raster_supported(int D, const Geometry& g) {
  // a copy segment (1 KiB) holds 1024 / (2 D) rows; they must be consecutive
  // raster rows, so the tile width must be a multiple of that count
  return fwd_bf16_supported(D, g) && g.w % (512 / D) == 0 && g.L / (512 / D) <= kMaxRasterSegs;
}

hipError_t launch_fwd_bf16_raster(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  uint16_t* o, float* lse, const Geometry& g, const HeadTable& ht,
                                  int B, int Hh, int D, float scale, hipStream_t st) {
  return launch_fwd_order<true>(q, k, v, o, lse, g, ht, B, Hh, D, scale, st);
}

hipError_t launch_mass_bf16(const uint16_t* q, const uint16_t* k, float* lse, const MassArgs& ma,
                            const Geometry& g, const HeadTable& ht_full, int B, int Hh, int D,
                            float scale, hipStream_t st) {
  const int L = g.L;
  const HeadTable& ht = ht_full;
  if (D == 128) {
    if (L % 128 == 0)
      return launch_cfg<128, 1, 4, 2, true>(q, k, k, nullptr, lse, g, ht, B, Hh, scale, st, ma);
    if (L % 64 == 0)
      return launch_cfg<128, 1, 2, 2, true>(q, k, k, nullptr, lse, g, ht, B, Hh, scale, st, ma);
    return launch_cfg<128, 1, 1, 1, true>(q, k, k, nullptr, lse, g, ht, B, Hh, scale, st, ma);
  }
  if (D == 64) {
    if (L % 128 == 0)
      return launch_cfg<64, 1, 4, 2, true>(q, k, k, nullptr, lse, g, ht, B, Hh, scale, st, ma);
    if (L % 64 == 0)
      return launch_cfg<64, 1, 2, 2, true>(q, k, k, nullptr, lse, g, ht, B, Hh, scale, st, ma);
    return launch_cfg<64, 1, 1, 1, true>(q, k, k, nullptr, lse, g, ht, B, Hh, scale, st, ma);
  }
  return hipErrorInvalidValue;
}

}  // namespace sta
