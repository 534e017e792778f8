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
//    padded latent get lse2 = +inf and Dl = 0: with finite scores every P of
//    such a query is then exactly zero, so the dK/dV passes need no query mask
//    and dQ is zero there by construction.
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
// PADM: 0 no padding; 1 padded latent with w = 8 and t*h <= 64 (row and column
// mask); 2 any other padded latent (a ballot per partial stage).
template <int D, int NW, int OCC, int PADM>
__global__ __launch_bounds__(64 * NW, OCC) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ dl, uint16_t* __restrict__ dq,
    Geometry g, HeadTable ht, int B, int Hh, float c_log2, float scale, int blocks_per_tile,
    int total, int group_items) {
  constexpr int KS = D / 16, DT = D / 32, TB = kStage * D * 2;
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

  const size_t row0 = seq + (size_t)qtile * g.L + sub * (NW * 32) + wave * 32;
  const size_t row = row0 + c32;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(q + row * D + ks * 16 + grp * 8));
  // The wave's 32 dO rows go to its LDS tile (the staged tiles' swizzle) and
  // are read back as the dP^T B operand each stage.
  char* dotile = dores + wave * TB;
  {
    constexpr int RPS = 1024 / (D * 2), CPR = D / 8;
    const int rin = lane / CPR, p = lane % CPR;
#pragma unroll
    for (int seg = 0; seg < 32 / RPS; ++seg) {
      const int r = seg * RPS + rin;
      dma16(dout + (row0 + r) * D + ((p ^ (int)swz<D>(r)) * 8), dotile + seg * 1024);
    }
  }
  const float lrow = lse2[row], ndrow = dl[row];  // -Dl

  const int a2 = qtile % g.n2, a1 = (qtile / g.n2) % g.n1, a0 = qtile / (g.n2 * g.n1);
  const int w0 = ht.wp[head][0], w1 = ht.wp[head][1], w2 = ht.wp[head][2];
  const int s0 = window_start(a0, w0, g.n0), s1 = window_start(a1, w1, g.n1),
            s2 = window_start(a2, w2, g.n2);
  const int spt = g.L / kStage;
  const int nst = w0 * w1 * w2 * spt;
  int i0 = 0, i1 = 0, i2 = 0, jb = 0;
  auto issue = [&](char* kl, char* vl) {
    const int key0 = (((s0 + i0) * g.n1 + (s1 + i1)) * g.n2 + (s2 + i2)) * g.L + jb * kStage;
    if (++jb == spt) {
      jb = 0;
      if (++i2 == w2) {
        i2 = 0;
        if (++i1 == w1) {
          i1 = 0;
          ++i0;
        }
      }
    }
    dma_kv<D, kStage, NW>(kb, vb, (size_t)key0, kl, vl, wave, lane);
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // Padded latents: keys at padding positions of a partial key tile get
  // P = 0 (a second walk over the key blocks, for the stage being computed).
  // The S^T accumulator holds key 8i + 4(l/32) + jj of the stage in element
  // 4i + jj: with w = 8 that is row 4 cjb + i of the tile and column
  // 4(l/32) + jj, so one bit per tile row (a ballot) and the tile's real width,
  // worked out once per key tile, mask a stage by adding 0 or -inf (scores are
  // finite, so the sum is exactly -inf).  PADM 2 tests every key of the block.
  int ci0 = 0, ci1 = 0, ci2 = 0, cjb = 0;
  bool key_tile_partial = false, col_partial = false;
  uint64_t rows_real = ~0ull;  // bit R: tile row R is real
  int col_ext = 8;             // real columns of the key tile
  auto mask_keys = [&](f32x16& st) {
    if constexpr (PADM == 0) return;
    const int k0 = s0 + ci0, k1 = s1 + ci1, k2 = s2 + ci2;
    if constexpr (PADM == 1) {
      if (cjb == 0) {  // a new key tile
        key_tile_partial = tile_partial(k0, k1, k2, g);
        if (key_tile_partial) {
          const int e0 = tile_ext(k0, g.t, g.T), e1 = tile_ext(k1, g.h, g.H), e2 = tile_ext(k2, g.w, g.W);
          const uint32_t r0 = fdiv((uint32_t)lane * 8u, g.fhw);  // lane / h (w = 8)
          const uint32_t r1 = (uint32_t)lane - r0 * (uint32_t)g.h;
          rows_real = __ballot(lane < g.t * g.h && (int)r0 < e0 && (int)r1 < e1);
          col_ext = e2;
          col_partial = e2 < 8;
        }
      }
      if (key_tile_partial) {
        const uint32_t rb = (uint32_t)(rows_real >> (4 * cjb)) & 0xfu;
        if (rb != 0xfu) {  // a row of the block is padding (uniform)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float rbias = (rb >> u) & 1u ? 0.f : -INFINITY;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) st[4 * u + jj] += rbias;
          }
        }
        if (col_partial) {
          float cb[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) cb[jj] = 4 * grp + jj < col_ext ? 0.f : -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; ++e) st[e] += cb[e & 3];
        }
      }
    } else if (tile_partial(k0, k1, k2, g)) {
      const uint32_t m = block_real_mask(k0, k1, k2, cjb * kStage, g, lane);
      if (m != 0xffffffffu) {
        const uint32_t bits = lane_bits(m, lane);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (!elem_real(bits, e)) st[e] = -INFINITY;
      }
    }
    if (++cjb == spt) {
      cjb = 0;
      if (++ci2 == w2) {
        ci2 = 0;
        if (++ci1 == w1) {
          ci1 = 0;
          ++ci0;
        }
      }
    }
  };

  auto step = [&](const char* kl, const char* vl) {
    bf16x8 kf[KS], vr[KS];
    read_rows<D>(kl, kf, grp, c32);
    read_rows<D>(vl, vr, grp, c32);
    f32x16 st = contract_rows<D>(kf, qf);         // S^T[key][q]
    mask_keys(st);
    // a scheduling boundary after the mask (the dP^T reads stay below it:
    // measured faster)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 dpt;
    {
      bf16x8 dof[KS];
      read_rows<D>(dotile, dof, grp, c32);
      dpt = contract_rows<D>(vr, dof);              // dP^T[key][q]
    }
    bf16x8 ds[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[8 * s + e], c_log2, -lrow));
        ds[s][e] = (__bf16)(p * (dpt[8 * s + e] + ndrow));
      }
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
  constexpr int PER = dma_kv_per_wave<D, kStage, NW>();
  issue(kl0, vl0);
  if (nst > 1) issue(kl1, vl1);
  wait_stage<PER>(nst > 1 ? 1 : 0);   // the dO tile and stage 0 have landed
  barrier_lds();
  // Both slots in one loop body with no exit in between (an exit there made
  // the compiler copy the accumulators every other stage); an odd last stage
  // runs after it.
  int j = 0;
  for (; j + 1 < nst; j += 2) {
    step(kl0, vl0);
    wait_dma();
    barrier_lds();
    if (j + 2 < nst) issue(kl0, vl0);
    step(kl1, vl1);
    if (j + 2 < nst) {
      wait_dma();
      barrier_lds();
      if (j + 3 < nst) issue(kl1, vl1);
    }
  }
  if (j < nst) step(kl0, vl0);

  // dQ = scale * dQ^T: lane holds query c32, d = dt*32 + 8i + 4g + jj; zero
  // on padding rows.
  const int rin = sub * (NW * 32) + wave * 32 + c32;  // row inside the query tile
  const float osc = (!g.padded || token_real(a0, a1, a2, rin, g)) ? scale : 0.0f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 w;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) w[jj] = (__bf16)(acc[dt][4 * i + jj] * osc);
      *(bf16x4*)(dq + row * D + dt * 32 + 8 * i + 4 * grp) = w;
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

// MODE 0 computes dV (S = Q K^T, P, dV += P^T dO); MODE 1 computes dK
// (S, dP = dO V^T, dS, dK += dS^T Q).  Two launches instead of one keep the
// resident state of each under the register file (one fused kernel spills).
template <int D, int NW, int MODE, int OCC>
__global__ __launch_bounds__(64 * NW, OCC) void bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse2, const float* __restrict__ dl, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, const int32_t* __restrict__ rank_tab, Geometry g, HeadTable ht,
    int B, int Hh, float c_log2, float scale, int blocks_per_tile) {
  constexpr int KS = D / 16, DT = D / 32, TB = kStage * D * 2;
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

  // Resident key rows: K^T as the B operand (lane holds 8 d of key c32); for
  // dK the wave's 32 V rows are copied into its LDS tile (swizzled like the
  // staged tiles) and read back per stage.
  const size_t krow0 = seq + (size_t)ktile * g.L + sub * (NW * 32) + wave * 32;
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kf[ks] = as_bf16x8(*(const u32x4*)(k + (krow0 + c32) * D + ks * 16 + grp * 8));
  char* vtile = vres + (MODE == 1 ? wave * TB : 0);
  if constexpr (MODE == 1) {
    constexpr int RPS = 1024 / (D * 2), CPR = D / 8;
    const int rin = lane / CPR, p = lane % CPR;
#pragma unroll
    for (int seg = 0; seg < 32 / RPS; ++seg) {
      const int r = seg * RPS + rin;
      dma16(v + (krow0 + r) * D + ((p ^ (int)swz<D>(r)) * 8), vtile + seg * 1024);
    }
  }

  // Query tiles whose window holds this key tile: a box [lo, hi] per dimension.
  const int a2 = ktile % g.n2, a1 = (ktile / g.n2) % g.n1, a0 = ktile / (g.n2 * g.n1);
  int lo0, hi0, lo1, hi1, lo2, hi2;
  window_transpose(a0, ht.wp[head][0], g.n0, &lo0, &hi0);
  window_transpose(a1, ht.wp[head][1], g.n1, &lo1, &hi1);
  window_transpose(a2, ht.wp[head][2], g.n2, &lo2, &hi2);
  const int c0 = hi0 - lo0 + 1, c1 = hi1 - lo1 + 1, c2 = hi2 - lo2 + 1;
  const int spt = g.L / kStage;
  const int nst = c0 * c1 * c2 * spt;
  int i0 = 0, i1 = 0, i2 = 0, jb = 0;
  auto issue = [&](char* ql, char* dol, char* st) {
    const size_t q0 =
        (size_t)(((lo0 + i0) * g.n1 + (lo1 + i1)) * g.n2 + (lo2 + i2)) * g.L + jb * kStage;
    if (++jb == spt) {
      jb = 0;
      if (++i2 == c2) {
        i2 = 0;
        if (++i1 == c1) {
          i1 = 0;
          ++i0;
        }
      }
    }
    dma_kv<D, kStage, NW>(qb, db, q0, ql, dol, wave, lane);
    dma_stats<D>(lse2, dl, seq + q0, st, wave, lane);
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // Padding queries of a padded latent need no mask here: their lse2 is +inf,
  // so their P (and dS) is exactly zero.
  auto step = [&](const char* ql, const char* dol, const char* st) {
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
      bf16x8 da[KS], vf[KS];
      read_rows<D>(dol, da, grp, c32);
      read_rows<D>(vtile, vf, grp, c32);
      // dP - Dl: the accumulation starts from -Dl of the element's query
      // (stage statistics, already in the accumulator's layout)
      f32x16 ndl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 d4 = *(const f32x4*)(st + 128 + (8 * i + 4 * grp) * 4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ndl[4 * i + jj] = d4[jj];
      }
      dp = contract_rows_from<D>(da, vf, ndl);  // dP[q][key] - Dl[q]
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
  issue(ql0, dol0, st0);
  wait_dma();
  barrier_lds();
  int j = 0;
  for (; j + 1 < nst; j += 2) {
    issue(ql1, dol1, st1);
    step(ql0, dol0, st0);
    wait_dma();
    barrier_lds();
    if (j + 2 < nst) issue(ql0, dol0, st0);
    step(ql1, dol1, st1);
    wait_dma();
    barrier_lds();
  }
  if (j < nst) step(ql0, dol0, st0);

  // dK = scale * acc or dV = acc: lane holds key 8i + 4g + jj, d = dt*32 + c32;
  // zero on padding rows.
  uint16_t* out = MODE == 0 ? dv : dk;
  const float osc = MODE == 0 ? 1.0f : scale;
  const uint32_t kbits =
      g.padded ? lane_bits(block_real_mask(a0, a1, a2, sub * (NW * 32) + wave * 32, g, lane), lane)
               : 0xffffffffu;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const size_t r = krow0 + 8 * (e >> 2) + 4 * grp + (e & 3);
      const __bf16 x = (__bf16)(elem_real(kbits, e) ? acc[dt][e] * osc : 0.0f);
      out[r * D + dt * 32 + c32] = __builtin_bit_cast(uint16_t, x);
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
  else if (g.w == 8 && g.t * g.h <= 64) dq_pass(std::integral_constant<int, 1>{});
  else dq_pass(std::integral_constant<int, 2>{});
  // dV asks for two waves per SIMD, except one-wave workgroups at D = 128,
  // whose registers allow one.
  hipLaunchKernelGGL((bwd_dkv_kernel<D, NW, 0, (NW >= 2 || D <= 64) ? 2 : 1>), dim3((uint32_t)total),
                     dim3(64 * NW), 0, st, q,
                     k, v, dout, lse2, dl, dk, dv, rank_tab, g, ht, B, Hh, c_log2, scale, bpt);
  // dK fits two waves per SIMD in 4-wave workgroups; smaller ones keep one.
  hipLaunchKernelGGL((bwd_dkv_kernel<D, NW, 1, NW >= 4 ? 2 : 1>), dim3((uint32_t)total), dim3(64 * NW), 0, st, q,
                     k, v, dout, lse2, dl, dk, dv, rank_tab, g, ht, B, Hh, c_log2, scale, bpt);
  return hipGetLastError();
}

}  // namespace

bool bwd_bf16_supported(int D, int L) { return (D == 64 || D == 128) && L % 32 == 0; }

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
