// STA backward, bf16 in/out, fp32 accumulation, on gfx950 MFMA.
//
// The gradient of the forward in fwd_bf16.hip ("Sliding Tile Attention",
// arXiv 2502.04507 summary page: the method is fine-tuned, which needs it).
// With P the window-masked softmax recomputed from the forward's LSE,
//   Dl_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - Dl_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
// Five launches, no atomics, deterministic:
//   0. rank:  per head, the key tiles in order of decreasing work (the number
//             of query tiles whose window holds them), for the key-major launch.
//   1. prep:  Dl and LSE * log2(e) per query row, into the workspace.
//   2. dQ:    query-tile-major, walking the window like the forward:
//             S^T = K Q^T, dP^T = V dO^T (lane = query), dQ^T += K^T dS^T.
//   3. dV and 4. dK: key-tile-major, walking the query tiles whose window
//             holds the key tile (an interval per dimension): S = Q K^T,
//             dP = dO V^T (lane = key), dV += P^T dO, dK += dS^T Q.  That count
//             varies several-fold between edge and centre tiles, so within
//             each head workgroups are launched heaviest first, heads one after
//             the other (cache locality), dealt round-robin to the XCDs.
// Every (query tile, key tile) pair is a full dense block, as in the forward.
// The operand layouts, LDS swizzle and transposed reads are those of
// mfma_common.h; a transposed read of a row-major [32 x D] tile gives the
// operand [d][row] with the row order of the accumulator (see fwd_bf16.hip).
#include <type_traits>

#include "kernels.h"
#include "mfma_common.h"

namespace sta {

namespace {

constexpr int kStage = 32;  // rows (keys or queries) per pipeline stage

// --------------------------------------------------------------------------
// 1. prep: Dl_i = <dO_i, O_i> (fp32) and lse2_i = LSE_i * log2(e).
//    D/8 lanes per row, 16-byte loads, shuffle reduction.  Padding rows of a
//    padded latent get lse2 = +inf and Dl = 0 (their P, dS and outputs are
//    also masked by selects in the passes below).
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ lse2,
                                                       float* __restrict__ dl, size_t rows,
                                                       Geometry g) {
  constexpr int LPR = D / 8;  // lanes per row
  const size_t row = ((size_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(o + row * D + c * 8);
    const u32x4 b = *(const u32x4*)(dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), s);
      s = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), s);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
  if (row < rows && c == 0) {
    bool real = true;
    if (g.padded) {
      const int r = (int)(row % (size_t)g.S), tile = r / g.L;
      const int a2 = tile % g.n2, a1 = (tile / g.n2) % g.n1, a0 = tile / (g.n2 * g.n1);
      real = token_real(a0, a1, a2, r - tile * g.L, g);
    }
    dl[row] = real ? -s : 0.f;  // -Dl: the dK pass starts its dP accumulation from it
    lse2[row] = real ? lse[row] * kLog2e : INFINITY;
  }
}

// --------------------------------------------------------------------------
// 0. rank: tab[head][r] = the key tile of rank r for that head, ranks ordered
//    by decreasing count of query tiles whose window holds the tile (ties by
//    tile number).  One workgroup per head; with more than kRankTiles tiles the
//    order is left as the identity.
// --------------------------------------------------------------------------
constexpr int kRankTiles = 8192;

__global__ __launch_bounds__(256) void bwd_rank_kernel(Geometry g, HeadTable ht,
                                                       int32_t* __restrict__ tab) {
  __shared__ int cost[kRankTiles];
  const int head = blockIdx.x, nt = g.ntiles;
  int32_t* out = tab + (size_t)head * nt;
  if (nt > kRankTiles) {
    for (int i = threadIdx.x; i < nt; i += 256) out[i] = i;
    return;
  }
  for (int i = threadIdx.x; i < nt; i += 256) {
    const int a2 = i % g.n2, a1 = (i / g.n2) % g.n1, a0 = i / (g.n2 * g.n1);
    int lo0, hi0, lo1, hi1, lo2, hi2;
    window_transpose(a0, ht.wp[head][0], g.n0, &lo0, &hi0);
    window_transpose(a1, ht.wp[head][1], g.n1, &lo1, &hi1);
    window_transpose(a2, ht.wp[head][2], g.n2, &lo2, &hi2);
    cost[i] = (hi0 - lo0 + 1) * (hi1 - lo1 + 1) * (hi2 - lo2 + 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt; i += 256) {
    const int ci = cost[i];
    int r = 0;
    for (int j = 0; j < nt; ++j) {
      const int cj = cost[j];
      r += (cj > ci) | ((cj == ci) & (j < i));
    }
    out[r] = i;
  }
}

// Key-major work item: items are (head slot, rank, batch, sub-block), head
// slowest: the workgroups running at one time belong to one or two heads and
// share those heads' Q and dO in the caches, and within a head the heaviest
// key tiles go first, so each head's light tiles fill the gaps while the next
// head starts.  Consecutive workgroups land on different XCDs (blockIdx
// round-robin).
struct KeyItem {
  int b, head, ktile, sub;
};
__device__ __forceinline__ KeyItem key_major_item(const int32_t* __restrict__ rank_tab, const Geometry& g,
                                                  const HeadTable& ht, int B, int Hh,
                                                  int blocks_per_tile) {
  uint32_t item = blockIdx.x;
  KeyItem it;
  it.sub = item % blocks_per_tile;
  item /= blocks_per_tile;
  it.b = item % B;
  item /= B;
  const int rank = item % g.ntiles;
  it.head = ht.order[item / g.ntiles];
  it.ktile = rank_tab[(size_t)it.head * g.ntiles + rank];
  return it;
}

// Work item decode shared by both kernels (see the forward for the XCD split).
__device__ __forceinline__ uint32_t work_item(int total, int group_items) {
  const uint32_t bid = blockIdx.x;
  const uint32_t xcd = bid & 7u, local = bid >> 3;
  if (group_items > 0) {
    const uint32_t per_x = (uint32_t)group_items >> 3;
    return (local / per_x) * (uint32_t)group_items + xcd * per_x + local % per_x;
  }
  const uint32_t per = (uint32_t)total >> 3, rem = (uint32_t)total & 7u;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Wait for the oldest in-flight stage copy while up to two newer stages (each
// PER copies per wave) stay in flight; `newer` is how many exist.
template <int PER>
__device__ __forceinline__ void wait_stage(int newer) {
  if (newer >= 2) wait_dma_upto<2 * PER>();
  else if (newer == 1) wait_dma_upto<PER>();
  else wait_dma();
}

template <int D>
__device__ __forceinline__ f32x16 contract_rows(const bf16x8 (&a)[D / 16], const bf16x8 (&b)[D / 16]) {
  f32x16 acc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) acc = mfma32(a[ks], b[ks], acc);
  return acc;
}
// The same contraction added to acc.
template <int D>
__device__ __forceinline__ f32x16 contract_rows_from(const bf16x8 (&a)[D / 16], const bf16x8 (&b)[D / 16],
                                                     f32x16 acc) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) acc = mfma32(a[ks], b[ks], acc);
  return acc;
}

// --------------------------------------------------------------------------
// 2. dQ (query-major).  Workgroup = NW waves x 32 query rows of one tile.
// --------------------------------------------------------------------------
// PADM: 0 whole-tile latent; 1 padded latent: the real query rows and keys of
// a partial tile are taken compacted, in the tile's (t, h, w) order with the
// padding positions left out (as in the forward), so only a partial key
// tile's last block can hold padding keys, at its end.
template <int D, int NW, int OCC, int PADM>
__global__ __launch_bounds__(64 * NW, OCC) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ dl, uint16_t* __restrict__ dq,
    Geometry g, HeadTable ht, int B, int Hh, float c_log2, float scale, int blocks_per_tile,
    int total, int group_items) {
  constexpr int KS = D / 16, DT = D / 32, TB = kStage * D * 2, ROWS = NW * 32;
  // Two-slot K/V ring plus a per-wave tile holding the wave's dO rows (64 KB
  // per 4-wave workgroup, so two fit a CU at two waves per SIMD).
  __shared__ __attribute__((aligned(1024))) char kl0[TB];
  __shared__ __attribute__((aligned(1024))) char vl0[TB];
  __shared__ __attribute__((aligned(1024))) char kl1[TB];
  __shared__ __attribute__((aligned(1024))) char vl1[TB];
  __shared__ __attribute__((aligned(1024))) char dores[NW * TB];

  uint32_t item = work_item(total, group_items);
  const int sub = item % blocks_per_tile;
  item /= blocks_per_tile;
  const int qtile = item % g.ntiles;
  item /= g.ntiles;
  const int b = item % B;
  const int head = ht.order[item / B];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 5, c32 = lane & 31;
  const size_t seq = ((size_t)b * Hh + head) * (size_t)g.S;
  const uint16_t* kb = k + seq * D;
  const uint16_t* vb = v + seq * D;
  const int a2 = qtile % g.n2, a1 = (qtile / g.n2) % g.n1, a0 = qtile / (g.n2 * g.n1);

  // The workgroup's query rows: compacted rows [sub * ROWS, (sub + 1) * ROWS)
  // of the tile; rows past its real count (padded latents) stand in with the
  // tile's first row, a real token, and their dQ is not written.
  int qn = g.L, qe1 = g.h, qe2 = g.w;
  float qinv1 = 1.0f, qinv2 = 1.0f;
  if constexpr (PADM != 0) {
    qe1 = tile_ext(a1, g.h, g.H);
    qe2 = tile_ext(a2, g.w, g.W);
    qn = tile_ext(a0, g.t, g.T) * qe1 * qe2;
    qinv1 = __builtin_amdgcn_rcpf((float)qe1);
    qinv2 = __builtin_amdgcn_rcpf((float)qe2);
  }
  auto qrow_of = [&](int c) -> size_t {  // row inside the sequence of compacted row c
    uint32_t r = (uint32_t)c;
    if (PADM != 0 && qn < g.L) {
      const TilePos tp = split_compact((uint32_t)c, qe1, qe2, qinv1, qinv2);
      r = c < qn ? (tp.t * (uint32_t)g.h + tp.h) * (uint32_t)g.w + tp.w : 0u;
    }
    return (size_t)qtile * g.L + r;
  };
  const int cw0 = sub * ROWS + wave * 32;  // the wave's first compacted row
  const bool qreal = PADM == 0 || cw0 + c32 < qn;
  const size_t row = seq + qrow_of(cw0 + c32);
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(q + row * D + ks * 16 + grp * 8));
  // The wave's 32 dO rows go to its LDS tile (the staged tiles' swizzle) and
  // are read from there once into the registers of the dP^T B operand.
  char* dotile = dores + wave * TB;
  {
    constexpr int RPS = 1024 / (D * 2), CPR = D / 8;
    const int rin = lane / CPR, p = lane % CPR;
#pragma unroll
    for (int seg = 0; seg < 32 / RPS; ++seg) {
      const int r = seg * RPS + rin;
      dma16(dout + (seq + qrow_of(cw0 + r)) * D + ((p ^ (int)swz<D>(r)) * 8), dotile + seg * 1024);
    }
  }
  const float lrow = lse2[row], ndrow = dl[row];  // -Dl
  // -Dl in every element: each stage's dP^T accumulation starts from this
  // block (the lane's query, hence its Dl, is the same for the whole walk),
  // so dS = P (dP - Dl) takes no subtraction.
  f32x16 ndl16;
#pragma unroll
  for (int e = 0; e < 16; ++e) ndl16[e] = ndrow;

  const int w0 = ht.wp[head][0], w1 = ht.wp[head][1], w2 = ht.wp[head][2];
  const int s0 = window_start(a0, w0, g.n0), s1 = window_start(a1, w1, g.n1),
            s2 = window_start(a2, w2, g.n2);
  const int spt = g.L / kStage;
  // Key blocks of the walk: L / 32 per whole key tile, ceil(real / 32) per
  // partial one (compacted), summed over the 8 classes of tiles (last along
  // t, h, w or not); none when the workgroup holds no real query row.
  auto tile_blocks = [&](int e0, int e1, int e2) -> int { return (e0 * e1 * e2 + kStage - 1) / kStage; };
  int nst = w0 * w1 * w2 * spt;
  if constexpr (PADM != 0) {
    const int x0 = tile_ext(g.n0 - 1, g.t, g.T), x1 = tile_ext(g.n1 - 1, g.h, g.H),
              x2 = tile_ext(g.n2 - 1, g.w, g.W);
    const int l0 = s0 + w0 == g.n0, l1 = s1 + w1 == g.n1, l2 = s2 + w2 == g.n2;
    nst = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int c0 = c & 1, c1 = (c >> 1) & 1, c2 = c >> 2;
      const int cnt = (c0 ? l0 : w0 - l0) * (c1 ? l1 : w1 - l1) * (c2 ? l2 : w2 - l2);
      nst += cnt * tile_blocks(c0 ? x0 : g.t, c1 ? x1 : g.h, c2 ? x2 : g.w);
    }
    if (sub * ROWS >= qn) nst = 0;
  }
  using Cp = KvDma<D, kStage, NW>;
  // lane offsets of the K/V copies worked out once (scalar base per issue)
  const Cp copier(__builtin_amdgcn_readfirstlane(wave), lane);
  // The walk's key tile, worked out when the walk enters it: its first row
  // and, with padding, its real extents, real key count and the reciprocals
  // of its real extents along h and w.
  int i0 = 0, i1 = 0, i2 = 0, jb = 0, kbt = spt;
  uint32_t korg = 0;
  int ke1 = g.h, ke2 = g.w, knreal = g.L;
  bool kpart = false;
  float kinv1 = 1.0f, kinv2 = 1.0f;
  auto enter_tile = [&]() __attribute__((always_inline)) {
    const int k0 = s0 + i0, k1 = s1 + i1, k2 = s2 + i2;
    korg = (uint32_t)(((k0 * g.n1 + k1) * g.n2 + k2) * g.L);
    if constexpr (PADM != 0) {
      const int e0 = tile_ext(k0, g.t, g.T);
      ke1 = tile_ext(k1, g.h, g.H);
      ke2 = tile_ext(k2, g.w, g.W);
      knreal = e0 * ke1 * ke2;
      kpart = knreal < g.L;
      kbt = tile_blocks(e0, ke1, ke2);
      if (kpart) {
        kinv1 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_amdgcn_rcpf((float)ke1))));
        kinv2 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_amdgcn_rcpf((float)ke2))));
      }
    }
  };
  enter_tile();
  // Copies the walk's next block into (kl, vl) and returns, for the stage
  // that computes it, its real key count when it ends a partial key tile
  // with padding (1..31), else 0.
  auto issue = [&](char* kl, char* vl) __attribute__((always_inline)) -> uint32_t {
    const uint32_t nv = jb == kbt - 1 ? (uint32_t)(knreal - jb * kStage) & (kStage - 1) : 0u;
    const uint32_t org = korg;
    const bool gather = PADM != 0 && kpart;
    uint32_t rel[Cp::PT];
    bool real[Cp::PT];
    if (gather) {
#pragma unroll
      for (int e = 0; e < Cp::PT; ++e) {
        const uint32_t c = (uint32_t)(jb * kStage) + copier.row_in_block(e, lane);
        const TilePos tp = split_compact(c, ke1, ke2, kinv1, kinv2);
        real[e] = c < (uint32_t)knreal;
        rel[e] = (tp.t * (uint32_t)g.h + tp.h) * (uint32_t)g.w + tp.w;
      }
    }
    const size_t key0 = (size_t)org + (size_t)(jb * kStage);
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
    if (gather)
      copier.issue_rows_gather(kb, vb, org, rel, real, kl, vl);
    else
      copier.issue(kb, vb, key0, kl, vl);
    return nv;
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // Padding keys: element 4i + jj of the S^T accumulator holds key
  // 8i + 4(l/32) + jj of the stage, so a stage whose block ends a partial key
  // tile sets dS of the keys at or past its real count nv to zero (a select,
  // so whatever the staged padding row holds gives exactly zero).
  auto mask_keys = [&](f32x16& x, uint32_t nv) {
    if constexpr (PADM != 0) {
      if (nv != 0u) {  // uniform
        const int n = (int)nv - 4 * grp;
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = 8 * (e >> 2) + (e & 3) < n ? x[e] : 0.0f;
      }
    }
  };

  bf16x8 dof[KS];  // the wave's dO rows (B operand of dP^T), read once from its tile
  auto step = [&](const char* kl, const char* vl, uint32_t nv) {
    bf16x8 kf[KS], vr[KS];
    read_rows<D>(kl, kf, grp, c32);
    read_rows<D>(vl, vr, grp, c32);
    f32x16 st = contract_rows<D>(kf, qf);         // S^T[key][q]
    // a scheduling boundary after S^T (measured faster)
    __builtin_amdgcn_sched_barrier(0);
    const f32x16 dpt = contract_rows_from<D>(vr, dof, ndl16);  // dP^T[key][q] - Dl[q]
    f32x16 dsf;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(st[e], c_log2, -lrow));
      dsf[e] = p * dpt[e];
    }
    mask_keys(dsf, nv);
    bf16x8 ds[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) ds[s][e] = (__bf16)dsf[8 * s + e];
    bf16x8 ktf[DT][2];
    read_cols<D>(kl, ktf, lane);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(ktf[dt][s], ds[s], acc[dt]);
  };

  // Two-stage LDS ring: stage j sits in slot j % 2; its copy is issued two
  // stages ahead, right after the barrier that ends stage j - 2 (every wave
  // has then finished reading that slot: each step consumes its reads).
  constexpr int PER = Cp::PER;  // copies per wave per stage
  uint32_t nv0 = 0, nv1 = 0;    // the real-key count of each slot's block
  if (nst > 0) nv0 = issue(kl0, vl0);
  if (nst > 1) nv1 = issue(kl1, vl1);
  wait_stage<PER>(nst > 1 ? 1 : 0);   // the dO tile and stage 0 have landed
  read_rows<D>(dotile, dof, grp, c32);  // the wave's own tile: no barrier needed
  barrier_lds();
  // Both slots in one loop body with no exit in between (an exit there made
  // the compiler copy the accumulators every other stage); an odd last stage
  // runs after it.
  int j = 0;
  for (; j + 1 < nst; j += 2) {
    step(kl0, vl0, nv0);
    wait_dma();
    barrier_lds();
    if (j + 2 < nst) nv0 = issue(kl0, vl0);
    step(kl1, vl1, nv1);
    if (j + 2 < nst) {
      wait_dma();
      barrier_lds();
      if (j + 3 < nst) nv1 = issue(kl1, vl1);
    }
  }
  if (j < nst) step(kl0, vl0, nv0);

  // dQ = scale * dQ^T: lane holds query c32, d = dt*32 + 8i + 4g + jj.  With
  // padding, a lane also writes zeros to the row at its uncompacted position
  // when that position is padding, so every row of the tile is written once.
  if constexpr (PADM != 0) {
    const int pos = cw0 + c32;  // uncompacted position in the tile
    if (!token_real(a0, a1, a2, pos, g)) {
      const size_t prow = seq + (size_t)qtile * g.L + pos;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) *(bf16x4*)(dq + prow * D + dt * 32 + 8 * i + 4 * grp) = bf16x4{};
    }
  }
  if (qreal) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = (__bf16)(acc[dt][4 * i + jj] * scale);
        *(bf16x4*)(dq + row * D + dt * 32 + 8 * i + 4 * grp) = w;
      }
  }
}

// --------------------------------------------------------------------------
// 3. dK / dV (key-major).  Workgroup = NW waves x 32 key rows of one tile.
// --------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void dma_stats(const float* __restrict__ lse2, const float* __restrict__ dl,
                                          size_t row0, char* stat, int wave, int lane) {
  // lanes 0-7 copy lse2[row0 .. row0+31], lanes 8-15 copy dl[...], into
  // stat[0..127] and stat[128..255].
  if (wave == 0 && lane < 16) {
    const float* src = lane < 8 ? lse2 + row0 + lane * 4 : dl + row0 + (lane - 8) * 4;
    dma16(src, stat);
  }
}

// The statistics of 32 arbitrary rows (a compacted block of a partial query
// tile): lane l < 32 copies lse2 of row rows(l) to stat[4 l], lane 32 + l
// copies dl of the same row to stat[128 + 4 l] (4-byte DMA, wave 0 only).
__device__ __forceinline__ void dma_stats_gather(const float* __restrict__ lse2, const float* __restrict__ dl,
                                                 size_t row, char* stat, int wave, int lane) {
  if (wave == 0) __builtin_amdgcn_global_load_lds(lane < 32 ? lse2 + row : dl + row, (lds_ptr_t)stat, 4, 0, 0);
}

// MODE 0 computes dV (S = Q K^T, P, dV += P^T dO); MODE 1 computes dK
// (S, dP = dO V^T, dS, dK += dS^T Q).  Two launches instead of one keep the
// resident state of each under the register file (one fused kernel spills).
// PADM as in the dQ pass: with padding the workgroup's key rows and the
// query blocks it walks are compacted, and only a partial query tile's last
// block can hold padding queries, at its end.
template <int D, int NW, int MODE, int OCC, int PADM>
__global__ __launch_bounds__(64 * NW, OCC) void bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ dl, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, const int32_t* __restrict__ rank_tab, Geometry g, HeadTable ht,
    int B, int Hh, float c_log2, float scale, int blocks_per_tile) {
  constexpr int KS = D / 16, DT = D / 32, TB = kStage * D * 2, ROWS = NW * 32;
  __shared__ __attribute__((aligned(1024))) char ql0[TB];
  __shared__ __attribute__((aligned(1024))) char dol0[TB];
  __shared__ __attribute__((aligned(1024))) char ql1[TB];
  __shared__ __attribute__((aligned(1024))) char dol1[TB];
  __shared__ __attribute__((aligned(256))) char st0[256];
  __shared__ __attribute__((aligned(256))) char st1[256];
  // dK: the workgroup's V rows stay in LDS (one 32-row tile per wave) rather
  // than in registers, which keeps the kernel at two waves per SIMD.
  __shared__ __attribute__((aligned(1024))) char vres[MODE == 1 ? NW * TB : 16];

  const KeyItem it = key_major_item(rank_tab, g, ht, B, Hh, blocks_per_tile);
  const int sub = it.sub, ktile = it.ktile, b = it.b, head = it.head;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 5, c32 = lane & 31;
  const size_t seq = ((size_t)b * Hh + head) * (size_t)g.S;
  const uint16_t* qb = q + seq * D;
  const uint16_t* db = dout + seq * D;
  const int a2 = ktile % g.n2, a1 = (ktile / g.n2) % g.n1, a0 = ktile / (g.n2 * g.n1);

  // The workgroup's key rows: compacted rows [sub * ROWS, (sub + 1) * ROWS)
  // of the key tile; rows past its real count (padded latents) stand in with
  // the tile's first row, a real token, and their dK, dV are not written.
  int kn = g.L, ke1 = g.h, ke2 = g.w;
  float kinv1 = 1.0f, kinv2 = 1.0f;
  if constexpr (PADM != 0) {
    ke1 = tile_ext(a1, g.h, g.H);
    ke2 = tile_ext(a2, g.w, g.W);
    kn = tile_ext(a0, g.t, g.T) * ke1 * ke2;
    kinv1 = __builtin_amdgcn_rcpf((float)ke1);
    kinv2 = __builtin_amdgcn_rcpf((float)ke2);
  }
  auto krow_of = [&](int c) -> size_t {  // row inside the sequence of compacted key row c
    uint32_t r = (uint32_t)c;
    if (PADM != 0 && kn < g.L) {
      const TilePos tp = split_compact((uint32_t)c, ke1, ke2, kinv1, kinv2);
      r = c < kn ? (tp.t * (uint32_t)g.h + tp.h) * (uint32_t)g.w + tp.w : 0u;
    }
    return (size_t)ktile * g.L + r;
  };
  const int cw0 = sub * ROWS + wave * 32;  // the wave's first compacted key row

  // Resident key rows: K^T as the B operand (lane holds 8 d of key c32); for
  // dK the wave's 32 V rows are copied into its LDS tile (swizzled like the
  // staged tiles) and read from there once into registers (vrow).
  const size_t krow = seq + krow_of(cw0 + c32);
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kf[ks] = as_bf16x8(*(const u32x4*)(k + krow * D + ks * 16 + grp * 8));
  char* vtile = vres + (MODE == 1 ? wave * TB : 0);
  bf16x8 vrow[MODE == 1 ? KS : 1];
  if constexpr (MODE == 1) {
    constexpr int RPS = 1024 / (D * 2), CPR = D / 8;
    const int rin = lane / CPR, p = lane % CPR;
#pragma unroll
    for (int seg = 0; seg < 32 / RPS; ++seg) {
      const int r = seg * RPS + rin;
      dma16(v + (seq + krow_of(cw0 + r)) * D + ((p ^ (int)swz<D>(r)) * 8), vtile + seg * 1024);
    }
  }

  // Query tiles whose window holds this key tile: a box [lo, hi] per dimension.
  int lo0, hi0, lo1, hi1, lo2, hi2;
  window_transpose(a0, ht.wp[head][0], g.n0, &lo0, &hi0);
  window_transpose(a1, ht.wp[head][1], g.n1, &lo1, &hi1);
  window_transpose(a2, ht.wp[head][2], g.n2, &lo2, &hi2);
  const int c0 = hi0 - lo0 + 1, c1 = hi1 - lo1 + 1, c2 = hi2 - lo2 + 1;
  const int spt = g.L / kStage;
  // Query blocks of the walk: L / 32 per whole query tile, ceil(real / 32)
  // per partial one, summed over the 8 classes of tiles (last along t, h, w
  // or not); none when the workgroup holds no real key row.
  auto tile_blocks = [&](int e0, int e1, int e2) -> int { return (e0 * e1 * e2 + kStage - 1) / kStage; };
  int nst = c0 * c1 * c2 * spt;
  if constexpr (PADM != 0) {
    const int x0 = tile_ext(g.n0 - 1, g.t, g.T), x1 = tile_ext(g.n1 - 1, g.h, g.H),
              x2 = tile_ext(g.n2 - 1, g.w, g.W);
    const int l0 = hi0 == g.n0 - 1, l1 = hi1 == g.n1 - 1, l2 = hi2 == g.n2 - 1;
    nst = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int e0 = c & 1, e1 = (c >> 1) & 1, e2 = c >> 2;
      const int cnt = (e0 ? l0 : c0 - l0) * (e1 ? l1 : c1 - l1) * (e2 ? l2 : c2 - l2);
      nst += cnt * tile_blocks(e0 ? x0 : g.t, e1 ? x1 : g.h, e2 ? x2 : g.w);
    }
    if (sub * ROWS >= kn) nst = 0;
  }
  using Cp = KvDma<D, kStage, NW>;
  // lane offsets of the Q/dO copies worked out once (scalar base per issue)
  const Cp copier(__builtin_amdgcn_readfirstlane(wave), lane);
  // The walk's query tile, worked out when the walk enters it: its first row
  // and, with padding, its real extents, real row count and the reciprocals
  // of its real extents along h and w.
  int i0 = 0, i1 = 0, i2 = 0, jb = 0, qbt = spt;
  uint32_t qorg = 0;
  int qe1 = g.h, qe2 = g.w, qnreal = g.L;
  bool qpart = false;
  float qinv1 = 1.0f, qinv2 = 1.0f;
  auto enter_tile = [&]() __attribute__((always_inline)) {
    const int t0 = lo0 + i0, t1 = lo1 + i1, t2 = lo2 + i2;
    qorg = (uint32_t)(((t0 * g.n1 + t1) * g.n2 + t2) * g.L);
    if constexpr (PADM != 0) {
      const int e0 = tile_ext(t0, g.t, g.T);
      qe1 = tile_ext(t1, g.h, g.H);
      qe2 = tile_ext(t2, g.w, g.W);
      qnreal = e0 * qe1 * qe2;
      qpart = qnreal < g.L;
      qbt = tile_blocks(e0, qe1, qe2);
      if (qpart) {
        qinv1 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_amdgcn_rcpf((float)qe1))));
        qinv2 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_amdgcn_rcpf((float)qe2))));
      }
    }
  };
  enter_tile();
  // Copies the walk's next query block (Q, dO and the rows' statistics) and
  // returns, for the stage that computes it, its real row count when it ends
  // a partial query tile with padding (1..31), else 0.
  auto issue = [&](char* ql, char* dol, char* st) __attribute__((always_inline)) -> uint32_t {
    const uint32_t nv = jb == qbt - 1 ? (uint32_t)(qnreal - jb * kStage) & (kStage - 1) : 0u;
    const uint32_t org = qorg;
    const bool gather = PADM != 0 && qpart;
    uint32_t rel[Cp::PT];
    bool real[Cp::PT];
    uint32_t srel = 0;  // the statistics row of this lane (lane % 32 of the block)
    if (gather) {
#pragma unroll
      for (int e = 0; e < Cp::PT; ++e) {
        const uint32_t c = (uint32_t)(jb * kStage) + copier.row_in_block(e, lane);
        const TilePos tp = split_compact(c, qe1, qe2, qinv1, qinv2);
        real[e] = c < (uint32_t)qnreal;
        rel[e] = (tp.t * (uint32_t)g.h + tp.h) * (uint32_t)g.w + tp.w;
      }
      const uint32_t c = (uint32_t)(jb * kStage) + (uint32_t)c32;
      const TilePos tp = split_compact(c, qe1, qe2, qinv1, qinv2);
      srel = c < (uint32_t)qnreal ? (tp.t * (uint32_t)g.h + tp.h) * (uint32_t)g.w + tp.w : 0u;
    }
    const size_t q0 = (size_t)org + (size_t)(jb * kStage);
    if (++jb == qbt) {
      jb = 0;
      if (++i2 == c2) {
        i2 = 0;
        if (++i1 == c1) {
          i1 = 0;
          ++i0;
        }
      }
      enter_tile();
    }
    if (gather) {
      copier.issue_rows_gather(qb, db, org, rel, real, ql, dol);
      dma_stats_gather(lse2, dl, seq + org + srel, st, wave, lane);
    } else {
      copier.issue(qb, db, q0, ql, dol);
      dma_stats<D>(lse2, dl, seq + q0, st, wave, lane);
    }
    return nv;
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // Padding queries: element 4i + jj of the S accumulator holds query
  // 8i + 4(l/32) + jj of the stage, so a stage whose block ends a partial
  // query tile sets the P (dV) or dS (dK) operand of the queries at or past
  // its real count nv to zero (a select, so whatever the staged padding row
  // holds contributes exactly nothing).
  auto mask_queries = [&](float (&x)[16], uint32_t nv) {
    if constexpr (PADM != 0) {
      if (nv != 0u) {  // uniform
        const int n = (int)nv - 4 * grp;
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = 8 * (e >> 2) + (e & 3) < n ? x[e] : 0.0f;
      }
    }
  };

  auto step = [&](const char* ql, const char* dol, const char* st, uint32_t nv) {
    f32x16 s, dp;
    {
      bf16x8 qa[KS];
      read_rows<D>(ql, qa, grp, c32);
      s = contract_rows<D>(qa, kf);   // S[q][key]
      // all Q-row reads first, then the MFMAs (left to itself the compiler
      // waits for the reads two at a time)
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);
    }
    if constexpr (MODE == 1) {
      bf16x8 da[KS];
      read_rows<D>(dol, da, grp, c32);
      // dP - Dl: the accumulation starts from -Dl of the element's query
      // (stage statistics, already in the accumulator's layout)
      f32x16 ndl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 d4 = *(const f32x4*)(st + 128 + (8 * i + 4 * grp) * 4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ndl[4 * i + jj] = d4[jj];
      }
      dp = contract_rows_from<D>(da, vrow, ndl);  // dP[q][key] - Dl[q]
    }
    // lane's queries: 8i + 4g + jj; the A operand is P^T (MODE 0) or dS^T.
    float pe[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *(const f32x4*)(st + (8 * i + 4 * grp) * 4);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int e = 4 * i + jj;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[e], c_log2, -l4[jj]));
        pe[e] = MODE == 0 ? p : p * dp[e];
      }
    }
    mask_queries(pe, nv);
    // the second GEMM's operand reads start after the exponentials (measured
    // faster for dV than the compiler's interleave; dK is indifferent)
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 af[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) af[e >> 3][e & 7] = (__bf16)pe[e];
    // B operand: dO^T (MODE 0) or Q^T, read transposed from the staged tile
    // (for dK, not hoisted above the vector work: registers are short).
    if constexpr (MODE == 1) __builtin_amdgcn_sched_barrier(0);
    bf16x8 bt[DT][2];
    read_cols<D>(MODE == 0 ? dol : ql, bt, lane);
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(af[ss], bt[dt][ss], acc[dt]);
    if constexpr (MODE == 0) {  // the same for the dO^T reads of dV (not dK: measured slower)
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * DT, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * DT, 1);
    }
  };

  // Two-stage LDS ring: the copy of stage j + 1 is issued before stage j is
  // computed.  Wave 0 also copies the stage statistics, so its waits cover one
  // more copy than the other waves'.
  // The loop body holds both slots and has no exit in between (an exit
  // there made the compiler copy the accumulators every other stage); an
  // odd last stage runs after it.
  uint32_t nv0 = 0, nv1 = 0;  // the real-row count of each slot's block
  if (nst > 0) nv0 = issue(ql0, dol0, st0);
  wait_dma();
  if constexpr (MODE == 1) read_rows<D>(vtile, vrow, grp, c32);  // the wave's own tile
  barrier_lds();
  int j = 0;
  for (; j + 1 < nst; j += 2) {
    nv1 = issue(ql1, dol1, st1);
    step(ql0, dol0, st0, nv0);
    wait_dma();
    barrier_lds();
    if (j + 2 < nst) nv0 = issue(ql0, dol0, st0);
    step(ql1, dol1, st1, nv1);
    wait_dma();
    barrier_lds();
  }
  if (j < nst) step(ql0, dol0, st0, nv0);

  // dK = scale * acc or dV = acc: lane holds key 8i + 4g + jj of the wave's
  // 32, d = dt*32 + c32.  With padding, keys past the real count are not
  // written, and each padding row of the tile gets zeros from the lane whose
  // uncompacted position it is.
  uint16_t* out = MODE == 0 ? dv : dk;
  const float osc = MODE == 0 ? 1.0f : scale;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int kk = cw0 + 8 * (e >> 2) + 4 * grp + (e & 3);  // compacted (and uncompacted) index
    if constexpr (PADM != 0) {
      if (!token_real(a0, a1, a2, kk, g)) {
        const size_t pr = seq + (size_t)ktile * g.L + kk;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) out[pr * D + dt * 32 + c32] = 0;
      }
      if (kk >= kn) continue;
    }
    const size_t r = seq + krow_of(kk);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      out[r * D + dt * 32 + c32] = __builtin_bit_cast(uint16_t, (__bf16)(acc[dt][e] * osc));
  }
}

inline int group_items_for(int seqs, int items_per_seq) {
  for (int gsz = 1; gsz <= 8; ++gsz)
    if ((gsz * items_per_seq) % 8 == 0 && seqs % gsz == 0) return gsz * items_per_seq;
  return 0;
}

template <int D, int NW>
hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk,
                      uint16_t* dv, float* ws, const Geometry& g, const HeadTable& ht, int B,
                      int Hh, float scale, hipStream_t st) {
  const size_t rows = (size_t)B * Hh * g.S;
  float* lse2 = ws;
  float* dl = ws + rows;
  int32_t* rank_tab = (int32_t*)(ws + 2 * rows);
  hipLaunchKernelGGL(bwd_rank_kernel, dim3((uint32_t)Hh), dim3(256), 0, st, g, ht, rank_tab);
  const size_t threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0,
                     st, o, dout, lse, lse2, dl, rows, g);
  const int bpt = g.L / (NW * 32);
  const int total = B * Hh * g.ntiles * bpt;
  const int group = group_items_for(B * Hh, g.ntiles * bpt);
  const float c_log2 = scale * kLog2e;
  // dQ fits two waves per SIMD in 4-wave workgroups; smaller ones keep one.
  // The padding mode is a template argument: mask code costs registers.
  auto dq_pass = [&](auto padm) {
    constexpr int PADM = decltype(padm)::value;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, NW >= 4 ? 2 : 1, PADM>), dim3((uint32_t)total), dim3(64 * NW), 0,
                       st, q, k, v, dout, lse2, dl, dq, g, ht, B, Hh, c_log2, scale, bpt, total, group);
  };
  if (!g.padded) dq_pass(std::integral_constant<int, 0>{});
  else dq_pass(std::integral_constant<int, 1>{});
  // dV asks for two waves per SIMD, except one-wave workgroups at D = 128,
  // whose registers allow one; dK fits two waves per SIMD in 4-wave
  // workgroups, smaller ones keep one.
  auto dkv_pass = [&](auto padm) {
    constexpr int PADM = decltype(padm)::value;
    hipLaunchKernelGGL((bwd_dkv_kernel<D, NW, 0, (NW >= 2 || D <= 64) ? 2 : 1, PADM>),
                       dim3((uint32_t)total), dim3(64 * NW), 0, st, q, k, v, dout, lse2, dl, dk, dv,
                       rank_tab, g, ht, B, Hh, c_log2, scale, bpt);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, NW, 1, NW >= 4 ? 2 : 1, PADM>), dim3((uint32_t)total),
                       dim3(64 * NW), 0, st, q, k, v, dout, lse2, dl, dk, dv, rank_tab, g, ht, B, Hh,
                       c_log2, scale, bpt);
  };
  if (!g.padded) dkv_pass(std::integral_constant<int, 0>{});
  else dkv_pass(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

}  // namespace

// A padded latent's compacted row index (below L) is split with fp32
// reciprocals, exact for indices below 2^21.
bool bwd_bf16_supported(int D, const Geometry& g) {
  return (D == 64 || D == 128) && g.L % 32 == 0 && (!g.padded || g.L <= (1 << 20));
}

hipError_t launch_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const uint16_t* dout, const float* lse,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, float* ws,
                           const Geometry& g, const HeadTable& ht, int B, int Hh, int D,
                           float scale, hipStream_t st) {
  // Workgroups of 4, 2 or 1 waves (32 rows each), the widest the tile allows.
  const int nw = g.L % 128 == 0 ? 4 : g.L % 64 == 0 ? 2 : 1;
  if (D == 128) {
    if (nw == 4) return launch_bwd<128, 4>(q, k, v, o, dout, lse, dq, dk, dv, ws, g, ht, B, Hh, scale, st);
    if (nw == 2) return launch_bwd<128, 2>(q, k, v, o, dout, lse, dq, dk, dv, ws, g, ht, B, Hh, scale, st);
    return launch_bwd<128, 1>(q, k, v, o, dout, lse, dq, dk, dv, ws, g, ht, B, Hh, scale, st);
  }
  if (D == 64) {
    if (nw == 4) return launch_bwd<64, 4>(q, k, v, o, dout, lse, dq, dk, dv, ws, g, ht, B, Hh, scale, st);
    if (nw == 2) return launch_bwd<64, 2>(q, k, v, o, dout, lse, dq, dk, dv, ws, g, ht, B, Hh, scale, st);
    return launch_bwd<64, 1>(q, k, v, o, dout, lse, dq, dk, dv, ws, g, ht, B, Hh, scale, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sta
