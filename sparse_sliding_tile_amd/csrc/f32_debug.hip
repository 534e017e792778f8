// fp32 debug instance of the STA forward and backward.
//
// Plain fp32 arithmetic (no MFMA, one thread per query or key row, K/V or Q/dO
// staged through LDS 32 rows at a time).  It exists to check the window walk
// and the softmax bookkeeping of the library at 1e-5 against the fp64 oracle;
// it is not a performance path.
#include "kernels.h"

namespace sta {

namespace {

constexpr int kRows = 128;  // threads (rows) per workgroup
constexpr int kChunk = 32;  // keys or queries staged per LDS round

struct TileCoord {
  int a0, a1, a2;
};

__device__ __forceinline__ TileCoord tile_coord(int a, const Geometry& g) {
  return {a / (g.n1 * g.n2), (a / g.n2) % g.n1, a % g.n2};
}

// Forward: O_i = sum_j softmax(scale q_i.k_j) v_j over the window's keys.
// LSE_ONLY computes the softmax normaliser alone (v and o are not touched).
template <int D, bool LSE_ONLY>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(const float* __restrict__ q,
                                                        const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        float* __restrict__ o,
                                                        float* __restrict__ lse, Geometry g,
                                                        HeadTable ht, int Hh, float scale) {
  __shared__ float ks[kChunk][D];
  __shared__ float vs[kChunk][D];
  const int subs = (g.L + kRows - 1) / kRows;
  int id = blockIdx.x;
  const int sub = id % subs;
  id /= subs;
  const int qt = id % g.ntiles;
  id /= g.ntiles;
  const int hh = id % Hh;
  const int b = id / Hh;
  const size_t base = ((size_t)b * Hh + hh) * (size_t)g.S * D;
  const int r = sub * kRows + threadIdx.x;
  const bool active = r < g.L;
  const size_t row = (size_t)qt * g.L + (active ? r : 0);

  float qv[D], acc[LSE_ONLY ? 1 : D];
  for (int d = 0; d < D; ++d) qv[d] = q[base + row * D + d];
  if constexpr (!LSE_ONLY)
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const TileCoord c = tile_coord(qt, g);
  const int w0 = ht.wp[hh][0], w1 = ht.wp[hh][1], w2 = ht.wp[hh][2];
  const int s0 = window_start(c.a0, w0, g.n0), s1 = window_start(c.a1, w1, g.n1),
            s2 = window_start(c.a2, w2, g.n2);
  for (int i0 = 0; i0 < w0; ++i0)
    for (int i1 = 0; i1 < w1; ++i1)
      for (int i2 = 0; i2 < w2; ++i2) {
        const int k0 = s0 + i0, k1 = s1 + i1, k2 = s2 + i2;
        const int kt = (k0 * g.n1 + k1) * g.n2 + k2;
        for (int j0 = 0; j0 < g.L; j0 += kChunk) {
          const int nk = min(kChunk, g.L - j0);
          __syncthreads();
          for (int x = threadIdx.x; x < nk * D; x += kRows) {
            const size_t kr = (size_t)kt * g.L + j0 + x / D;
            ks[x / D][x % D] = k[base + kr * D + x % D];
            if constexpr (!LSE_ONLY) vs[x / D][x % D] = v[base + kr * D + x % D];
          }
          __syncthreads();
          float s[kChunk];
          float mc = -INFINITY;
          for (int j = 0; j < kChunk; ++j) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(qv[d], ks[j][d], dot);
            const bool key = j < nk && (!g.padded || token_real(k0, k1, k2, j0 + j, g));
            s[j] = key ? dot * scale : -INFINITY;
            mc = fmaxf(mc, s[j]);
          }
          const float mn = fmaxf(m, mc);
          const float corr = expf(m - mn);
          l *= corr;
          if constexpr (!LSE_ONLY)
            for (int d = 0; d < D; ++d) acc[d] *= corr;
          for (int j = 0; j < nk; ++j) {
            const float p = expf(s[j] - mn);  // 0 for a masked key
            l += p;
            if constexpr (!LSE_ONLY)
              for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
          }
          m = mn;
        }
      }
  if (!active) return;
  // Padding rows (padded latents) are no query: zero output.
  const bool real = !g.padded || token_real(c.a0, c.a1, c.a2, r, g);
  if constexpr (!LSE_ONLY) {
    const float inv = real ? 1.f / l : 0.f;
    for (int d = 0; d < D; ++d) o[base + row * D + d] = acc[d] * inv;
  }
  if (lse) lse[((size_t)b * Hh + hh) * g.S + row] = real ? m + logf(l) : 0.f;
}

// Dl_i = <dO_i, O_i>, one thread per row.
template <int D>
__global__ __launch_bounds__(256) void dl_f32_kernel(const float* __restrict__ o,
                                                     const float* __restrict__ dout,
                                                     float* __restrict__ dl, size_t rows) {
  const size_t r = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float s = 0.f;
  for (int d = 0; d < D; ++d) s = fmaf(dout[r * D + d], o[r * D + d], s);
  dl[r] = s;
}

// dQ_i = scale sum_j P_ij (<dO_i, v_j> - Dl_i) k_j over the window's keys.
template <int D>
__global__ __launch_bounds__(kRows) void dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dl,
    float* __restrict__ dq, Geometry g, HeadTable ht, int Hh, float scale) {
  __shared__ float ks[kChunk][D];
  __shared__ float vs[kChunk][D];
  const int subs = (g.L + kRows - 1) / kRows;
  int id = blockIdx.x;
  const int sub = id % subs;
  id /= subs;
  const int qt = id % g.ntiles;
  id /= g.ntiles;
  const int hh = id % Hh;
  const int b = id / Hh;
  const size_t bh = (size_t)b * Hh + hh;
  const size_t base = bh * (size_t)g.S * D;
  const int r = sub * kRows + threadIdx.x;
  const bool active = r < g.L;
  const size_t row = (size_t)qt * g.L + (active ? r : 0);

  float qv[D], dov[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = q[base + row * D + d];
    dov[d] = dout[base + row * D + d];
    acc[d] = 0.f;
  }
  const float li = lse[bh * g.S + row], di = dl[bh * g.S + row];

  const TileCoord c = tile_coord(qt, g);
  const int w0 = ht.wp[hh][0], w1 = ht.wp[hh][1], w2 = ht.wp[hh][2];
  const int s0 = window_start(c.a0, w0, g.n0), s1 = window_start(c.a1, w1, g.n1),
            s2 = window_start(c.a2, w2, g.n2);
  for (int i0 = 0; i0 < w0; ++i0)
    for (int i1 = 0; i1 < w1; ++i1)
      for (int i2 = 0; i2 < w2; ++i2) {
        const int k0 = s0 + i0, k1 = s1 + i1, k2 = s2 + i2;
        const int kt = (k0 * g.n1 + k1) * g.n2 + k2;
        for (int j0 = 0; j0 < g.L; j0 += kChunk) {
          const int nk = min(kChunk, g.L - j0);
          __syncthreads();
          for (int x = threadIdx.x; x < nk * D; x += kRows) {
            const size_t kr = (size_t)kt * g.L + j0 + x / D;
            ks[x / D][x % D] = k[base + kr * D + x % D];
            vs[x / D][x % D] = v[base + kr * D + x % D];
          }
          __syncthreads();
          for (int j = 0; j < nk; ++j) {
            if (g.padded && !token_real(k0, k1, k2, j0 + j, g)) continue;  // padding key
            float s = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
              s = fmaf(qv[d], ks[j][d], s);
              dp = fmaf(dov[d], vs[j][d], dp);
            }
            const float p = expf(s * scale - li);
            const float ds = p * (dp - di) * scale;
            for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, ks[j][d], acc[d]);
          }
        }
      }
  if (!active) return;
  const bool real = !g.padded || token_real(c.a0, c.a1, c.a2, r, g);
  for (int d = 0; d < D; ++d) dq[base + row * D + d] = real ? acc[d] : 0.f;
}

// dK_j = scale sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i over the query tiles
// whose window holds key tile kt.
template <int D>
__global__ __launch_bounds__(kRows) void dkv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dl,
    float* __restrict__ dk, float* __restrict__ dv, Geometry g, HeadTable ht, int Hh,
    float scale) {
  __shared__ float qs[kChunk][D];
  __shared__ float dos[kChunk][D];
  __shared__ float ls[kChunk], ds_[kChunk];
  const int subs = (g.L + kRows - 1) / kRows;
  int id = blockIdx.x;
  const int sub = id % subs;
  id /= subs;
  const int kt = id % g.ntiles;
  id /= g.ntiles;
  const int hh = id % Hh;
  const int b = id / Hh;
  const size_t bh = (size_t)b * Hh + hh;
  const size_t base = bh * (size_t)g.S * D;
  const int r = sub * kRows + threadIdx.x;
  const bool active = r < g.L;
  const size_t row = (size_t)kt * g.L + (active ? r : 0);

  float kv[D], vv[D], ak[D], av[D];
  for (int d = 0; d < D; ++d) {
    kv[d] = k[base + row * D + d];
    vv[d] = v[base + row * D + d];
    ak[d] = 0.f;
    av[d] = 0.f;
  }
  const TileCoord c = tile_coord(kt, g);
  int l0, h0, l1, h1, l2, h2;
  window_transpose(c.a0, ht.wp[hh][0], g.n0, &l0, &h0);
  window_transpose(c.a1, ht.wp[hh][1], g.n1, &l1, &h1);
  window_transpose(c.a2, ht.wp[hh][2], g.n2, &l2, &h2);
  for (int q0 = l0; q0 <= h0; ++q0)
    for (int q1 = l1; q1 <= h1; ++q1)
      for (int q2 = l2; q2 <= h2; ++q2) {
        const int qt = (q0 * g.n1 + q1) * g.n2 + q2;
        for (int i0 = 0; i0 < g.L; i0 += kChunk) {
          const int nq = min(kChunk, g.L - i0);
          __syncthreads();
          for (int x = threadIdx.x; x < nq * D; x += kRows) {
            const size_t qr = (size_t)qt * g.L + i0 + x / D;
            qs[x / D][x % D] = q[base + qr * D + x % D];
            dos[x / D][x % D] = dout[base + qr * D + x % D];
          }
          if (threadIdx.x < nq) {
            ls[threadIdx.x] = lse[bh * g.S + (size_t)qt * g.L + i0 + threadIdx.x];
            ds_[threadIdx.x] = dl[bh * g.S + (size_t)qt * g.L + i0 + threadIdx.x];
          }
          __syncthreads();
          for (int i = 0; i < nq; ++i) {
            if (g.padded && !token_real(q0, q1, q2, i0 + i, g)) continue;  // padding query
            float s = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
              s = fmaf(qs[i][d], kv[d], s);
              dp = fmaf(dos[i][d], vv[d], dp);
            }
            const float p = expf(s * scale - ls[i]);
            const float dsc = p * (dp - ds_[i]) * scale;
            for (int d = 0; d < D; ++d) {
              av[d] = fmaf(p, dos[i][d], av[d]);
              ak[d] = fmaf(dsc, qs[i][d], ak[d]);
            }
          }
        }
      }
  if (!active) return;
  const bool real = !g.padded || token_real(c.a0, c.a1, c.a2, r, g);
  for (int d = 0; d < D; ++d) {
    dk[base + row * D + d] = real ? ak[d] : 0.f;
    dv[base + row * D + d] = real ? av[d] : 0.f;
  }
}

template <int D>
hipError_t fwd_f32_d(const float* q, const float* k, const float* v, float* o, float* lse,
                     const Geometry& g, const HeadTable& ht, int B, int Hh, float scale,
                     hipStream_t st) {
  const int subs = (g.L + kRows - 1) / kRows;
  const dim3 grid((uint32_t)(B * Hh * g.ntiles * subs));
  if (o == nullptr)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), grid, dim3(kRows), 0, st, q, k, v, o, lse, g, ht,
                       Hh, scale);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), grid, dim3(kRows), 0, st, q, k, v, o, lse, g,
                       ht, Hh, scale);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_f32_d(const float* q, const float* k, const float* v, const float* o,
                     const float* dout, const float* lse, float* dq, float* dk, float* dv,
                     float* dl, const Geometry& g, const HeadTable& ht, int B, int Hh, float scale,
                     hipStream_t st) {
  const size_t rows = (size_t)B * Hh * g.S;
  hipLaunchKernelGGL((dl_f32_kernel<D>), dim3((uint32_t)((rows + 255) / 256)), dim3(256), 0, st, o,
                     dout, dl, rows);
  const int subs = (g.L + kRows - 1) / kRows;
  const dim3 grid((uint32_t)(B * Hh * g.ntiles * subs));
  hipLaunchKernelGGL((dq_f32_kernel<D>), grid, dim3(kRows), 0, st, q, k, v, dout, lse, dl, dq, g,
                     ht, Hh, scale);
  hipLaunchKernelGGL((dkv_f32_kernel<D>), grid, dim3(kRows), 0, st, q, k, v, dout, lse, dl, dk,
                     dv, g, ht, Hh, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const Geometry& g, const HeadTable& ht, int B, int Hh, int D,
                          float scale, hipStream_t st) {
  switch (D) {
    case 32: return fwd_f32_d<32>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    case 64: return fwd_f32_d<64>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    case 128: return fwd_f32_d<128>(q, k, v, o, lse, g, ht, B, Hh, scale, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* dl, const Geometry& g, const HeadTable& ht, int B, int Hh, int D,
                          float scale, hipStream_t st) {
  switch (D) {
    case 32: return bwd_f32_d<32>(q, k, v, o, dout, lse, dq, dk, dv, dl, g, ht, B, Hh, scale, st);
    case 64: return bwd_f32_d<64>(q, k, v, o, dout, lse, dq, dk, dv, dl, g, ht, B, Hh, scale, st);
    case 128:
      return bwd_f32_d<128>(q, k, v, o, dout, lse, dq, dk, dv, dl, g, ht, B, Hh, scale, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sta
