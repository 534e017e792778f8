// STA forward, bf16 in/out, fp32 accumulation, on gfx950 MFMA.
//
// "Sliding Tile Attention" (arXiv 2502.04507 summary page, abstract and method
// details): each query tile attends densely to the key tiles of its window, so
// every (query block, key block) product below is a full dense contraction and
// there is no mask anywhere in the inner loop.
//
// Work decomposition
//   One workgroup = NW waves = NW*QT*32 query rows of one query tile of one
//   (batch, head).  Each wave keeps its QT*32 query rows resident in registers
//   for the whole key walk.  The key tiles of the window are walked in KB-key
//   blocks, double-buffered through LDS (K row-major, V transposed), loaded with
//   16-byte global loads.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, A: 32x16, B: 16x32, C: 32x32)
//   S^T = K Q^T   A = K rows from LDS, B = Q^T from registers; lane l of the
//                 accumulator holds query (l % 32) and 16 keys, so the softmax
//                 row statistics are per-lane scalars (plus one exchange with
//                 lane l ^ 32).
//   O^T += V^T P^T  A = V^T from LDS, B = P^T straight from the S^T accumulator
//                 (converted to bf16); lane l keeps query (l % 32) again, so the
//                 output rescale and the final 1/l are per-lane scalars.
//   The key order inside each 16-key MFMA step follows the accumulator layout
//   (key bits 2 and 3 swapped); V^T is written to LDS in that order.
//
// Softmax: scores are scaled by scale*log2(e) inside one FMA and exponentiated
// with exp2.  The running maximum is only raised (and O, l rescaled) when a
// block's maximum exceeds it by more than 8 (a factor 256), which keeps every
// probability below 256 and is exact in real arithmetic since O and l are
// always scaled by the same factor.
#include "kernels.h"

namespace sta {

namespace {

constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Byte offset of 16-byte chunk c of row r in an LDS array with CH chunks per
// row, XOR-swizzled so that 8 consecutive rows read at one chunk position hit
// 8 distinct 4-bank groups.
template <int CH>
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t c) {
  uint32_t p;
  if constexpr (CH >= 8) {
    p = c ^ ((r ^ (r >> 3)) & 7);
  } else if constexpr (CH == 4) {
    p = c ^ ((r >> 1) & 3);
  } else {
    p = c ^ ((r >> 2) & 1);
  }
  return r * (CH * 16) + p * 16;
}

// Position of key kk (0..31 inside a 32-key sub-tile) in the V^T LDS rows:
// bits 2 and 3 swapped, matching the accumulator order of S^T.
__device__ __forceinline__ uint32_t vslot(uint32_t kk) {
  return (kk & 0x13u) | ((kk & 4u) << 1) | ((kk & 8u) >> 1);
}

__device__ __forceinline__ float wave_swap32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Packs the bf16 of element e of four (or two) key rows into the (key-major)
// 8- (or 4-) byte group written to one V^T row.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // (a.lo, b.lo)
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // (a.hi, b.hi)
}

template <int D, int QT, int NW, int KB>
struct FwdCfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWS = NW * QT * 32;  // query rows per workgroup
  static constexpr int KS = D / 16;          // MFMA k-steps of Q K^T
  static constexpr int DT = D / 32;          // 32-wide d tiles of O^T
  static constexpr int KT = KB / 32;         // 32-key sub-tiles per block
  static constexpr int KCH = D / 8;          // 16-byte chunks per K row
  static constexpr int VCH = KB / 8;         // 16-byte chunks per V^T row
  static constexpr int KBYTES = KB * D * 2;  // one K (or V^T) block in LDS
  // K load: 16-byte chunks per thread.
  static constexpr int KLOADS = KB * KCH / THREADS;
  // V load: units of KG keys x 8 d per thread.
  static constexpr int KG = (KB / 4) * KCH >= THREADS ? 4 : 2;
  static constexpr int VUNITS = (KB / KG) * KCH / THREADS;
  static_assert(KLOADS >= 1 && KB * KCH % THREADS == 0, "K block does not split over threads");
  static_assert(VUNITS >= 1 && (KB / KG) * KCH % THREADS == 0, "V block does not split");
};

template <int D, int QT, int NW, int KB>
__global__ __launch_bounds__(64 * NW) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse, Geometry g,
    HeadTable ht, int B, int Hh, float c_log2, int blocks_per_tile, int total) {
  using C = FwdCfg<D, QT, NW, KB>;
  __shared__ __attribute__((aligned(16))) char smem[2][2][C::KBYTES];

  // ---- work item: XCD-aware contiguous ranges (workgroups go round-robin to
  // the 8 XCDs, so XCD x gets every 8th blockIdx; remap so that it walks one
  // contiguous run of (head, query tile) items and its L2 sees neighbouring
  // windows).
  const uint32_t bid = blockIdx.x;
  const uint32_t xcd = bid & 7u, local = bid >> 3;
  const uint32_t per = (uint32_t)total >> 3, rem = (uint32_t)total & 7u;
  uint32_t item = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int sub = item % blocks_per_tile;
  item /= blocks_per_tile;
  const int qtile = item % g.ntiles;
  item /= g.ntiles;
  const int b = item % B;
  const int hslot = item / B;
  const int head = ht.order[hslot];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 5, c32 = lane & 31;

  const size_t seq = ((size_t)b * Hh + head) * (size_t)g.S;
  const uint16_t* qb = q + seq * D;
  const uint16_t* kb = k + seq * D;
  const uint16_t* vb = v + seq * D;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds 8 d of its row.
  const int qrow0 = qtile * g.L + sub * C::ROWS + wave * QT * 32;
  bf16x8 qf[QT][C::KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[qt][ks] = as_bf16x8(*(const u32x4*)(qb + (size_t)(qrow0 + qt * 32 + c32) * D +
                                                ks * 16 + grp * 8));

  // ---- window of this query tile
  const int a2 = qtile % g.n2, a1 = (qtile / g.n2) % g.n1, a0 = qtile / (g.n2 * g.n1);
  const int w0 = ht.wp[head][0], w1 = ht.wp[head][1], w2 = ht.wp[head][2];
  const int s0 = window_start(a0, w0, g.n0), s1 = window_start(a1, w1, g.n1),
            s2 = window_start(a2, w2, g.n2);
  const int bpt = g.L / KB;  // key blocks per key tile
  const int nblk = w0 * w1 * w2 * bpt;

  // Key-block walk state (incremented, no divisions in the loop).
  int i0 = 0, i1 = 0, i2 = 0, jb = 0;
  auto block_key0 = [&]() -> int {
    return (((s0 + i0) * g.n1 + (s1 + i1)) * g.n2 + (s2 + i2)) * g.L + jb * KB;
  };
  auto advance = [&]() {
    if (++jb == bpt) {
      jb = 0;
      if (++i2 == w2) {
        i2 = 0;
        if (++i1 == w1) {
          i1 = 0;
          ++i0;
        }
      }
    }
  };

  // ---- global -> register staging of one K/V block
  u32x4 kreg[C::KLOADS];
  u32x4 vreg[C::VUNITS][C::KG];
  auto load_block = [&](int key0) {
#pragma unroll
    for (int e = 0; e < C::KLOADS; ++e) {
      const int z = tid + e * C::THREADS;
      const int row = z / C::KCH, cc = z % C::KCH;
      kreg[e] = *(const u32x4*)(kb + (size_t)(key0 + row) * D + cc * 8);
    }
#pragma unroll
    for (int e = 0; e < C::VUNITS; ++e) {
      const int u = tid + e * C::THREADS;
      const int cc = u % C::KCH, kg = u / C::KCH;
#pragma unroll
      for (int j = 0; j < C::KG; ++j)
        vreg[e][j] = *(const u32x4*)(vb + (size_t)(key0 + kg * C::KG + j) * D + cc * 8);
    }
  };
  auto store_block = [&](int buf) {
    char* kl = smem[buf][0];
    char* vl = smem[buf][1];
#pragma unroll
    for (int e = 0; e < C::KLOADS; ++e) {
      const int z = tid + e * C::THREADS;
      const int row = z / C::KCH, cc = z % C::KCH;
      *(u32x4*)(kl + swz<C::KCH>(row, cc)) = kreg[e];
    }
#pragma unroll
    for (int e = 0; e < C::VUNITS; ++e) {
      const int u = tid + e * C::THREADS;
      const int cc = u % C::KCH, kg = u / C::KCH;
      const int key = kg * C::KG;                        // first key of the group
      const int slot = (key & ~31) | (int)vslot(key & 31);  // KG keys stay adjacent
      const int chunk = slot >> 3, within = (slot & 7) * 2;
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {  // d pair (2dw, 2dw+1) of this chunk
        const int d_lo = cc * 8 + 2 * dw;
        if constexpr (C::KG == 4) {
          u32x2 lo, hi;
          lo.x = pack_lo(vreg[e][0][dw], vreg[e][1][dw]);
          lo.y = pack_lo(vreg[e][2][dw], vreg[e][3][dw]);
          hi.x = pack_hi(vreg[e][0][dw], vreg[e][1][dw]);
          hi.y = pack_hi(vreg[e][2][dw], vreg[e][3][dw]);
          *(u32x2*)(vl + swz<C::VCH>(d_lo, chunk) + within) = lo;
          *(u32x2*)(vl + swz<C::VCH>(d_lo + 1, chunk) + within) = hi;
        } else {
          *(uint32_t*)(vl + swz<C::VCH>(d_lo, chunk) + within) =
              pack_lo(vreg[e][0][dw], vreg[e][1][dw]);
          *(uint32_t*)(vl + swz<C::VCH>(d_lo + 1, chunk) + within) =
              pack_hi(vreg[e][0][dw], vreg[e][1][dw]);
        }
      }
    }
  };

  // ---- accumulators
  f32x16 oacc[QT][C::DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qt][dt][e] = 0.f;
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
  }

  load_block(block_key0());
  advance();
  store_block(0);
  __syncthreads();

  for (int blk = 0; blk < nblk; ++blk) {
    const int buf = blk & 1;
    const bool more = blk + 1 < nblk;
    if (more) {
      load_block(block_key0());
      advance();
    }
    const char* kl = smem[buf][0];
    const char* vl = smem[buf][1];

    // S^T = K Q^T for the KT sub-tiles of this block.
    f32x16 sacc[C::KT][QT];
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kt][qt][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = as_bf16x8(*(const u32x4*)(kl + swz<C::KCH>(kt * 32 + c32, ks * 2 + grp)));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qt][ks], sacc[kt][qt], 0, 0, 0);
      }
    }

    // Online softmax (lazy rescale).
    bool need = false;
    float mblk[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = sacc[0][qt][0];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kt][qt][e]);
      mx = fmaxf(mx, wave_swap32(mx));
      mblk[qt] = mx * c_log2;
      need |= mblk[qt] > mrun[qt] + kRescaleThreshold;
    }
    if (__any(need)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mn = fmaxf(mrun[qt], mblk[qt]);
        const float alpha = __builtin_amdgcn_exp2f(mrun[qt] - mn);
        mrun[qt] = mn;
        lrun[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[qt][dt][e] *= alpha;
      }
    }
    bf16x8 pf[QT][C::KT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float mneg = -mrun[qt];
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][qt][8 * s + e], c_log2, mneg));
            ls += p;
            pf[qt][kt][s][e] = (__bf16)p;
          }
        }
      lrun[qt] += ls;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 a =
              as_bf16x8(*(const u32x4*)(vl + swz<C::VCH>(dt * 32 + c32, kt * 4 + s * 2 + grp)));
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            oacc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qt][kt][s], oacc[qt][dt], 0, 0, 0);
        }

    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = lrun[qt] + wave_swap32(lrun[qt]);
    const float inv = 1.0f / lt;
    const size_t row = (size_t)(qrow0 + qt * 32 + c32);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[qt][dt][4 * i + j] * inv);
        *(bf16x4*)(o + seq * D + row * D + dt * 32 + 8 * i + 4 * grp) = w;
      }
    if (lse != nullptr && grp == 0) lse[seq + row] = (mrun[qt] + log2f(lt)) * kLn2;
  }
}

template <int D, int QT, int NW, int KB>
hipError_t launch_cfg(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                      float* lse, const Geometry& g, const HeadTable& ht, int B, int Hh,
                      float scale, hipStream_t st) {
  using C = FwdCfg<D, QT, NW, KB>;
  const int bpt = g.L / C::ROWS;
  const int total = B * Hh * g.ntiles * bpt;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QT, NW, KB>), dim3((uint32_t)total), dim3(C::THREADS), 0,
                     st, q, k, v, o, lse, g, ht, B, Hh, scale * kLog2e, bpt, total);
  return hipGetLastError();
}

}  // namespace

bool fwd_bf16_supported(int D, int L) { return (D == 64 || D == 128) && L % 32 == 0; }

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, const Geometry& g, const HeadTable& ht, int B, int Hh,
                           int D, float scale, hipStream_t st) {
  const int L = g.L;
  if (D == 128) {
    if (L % 128 == 0) return launch_cfg<128, 1, 4, 64>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    return launch_cfg<128, 1, 1, 32>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
  }
  if (D == 64) {
    if (L % 128 == 0) return launch_cfg<64, 1, 4, 64>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    return launch_cfg<64, 1, 1, 32>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sta
