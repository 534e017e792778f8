// Attention mass of a candidate window, per (batch, head).
//
// "Sliding Tile Attention" (arXiv 2502.04507 summary page, method details):
// the window is set per head, automatically.  The measurement behind that
// choice is how much of a head's full softmax attention a window keeps.  For
// query row i, the window's share of the full attention is
//   sum_{j in window} exp(s_ij) / sum_{all j} exp(s_ij) = exp(LSE_win,i - LSE_full,i),
// so only normalisers are needed.  The bf16 path gets every candidate's share
// per row from one pass of the forward kernel's mass instance (full window,
// one sum per candidate under a shared running maximum) and only the final
// mean is done here (mass_reduce_kernel); the fp32 debug path combines
// separate log-sum-exp passes: mass = mean over the real query rows of
// exp(LSE_win - LSE_full) (mass_kernel).
#include "kernels.h"

namespace sta {

namespace {

constexpr int kThreads = 256;

// One workgroup per (batch, head) sequence; a fixed-order fp64 tree sum, so
// the result does not depend on scheduling.
__global__ __launch_bounds__(kThreads) void mass_kernel(const float* __restrict__ lse_win,
                                                        const float* __restrict__ lse_full,
                                                        float* __restrict__ mass, Geometry g,
                                                        double inv_real) {
  __shared__ double part[kThreads];
  const size_t base = (size_t)blockIdx.x * g.S;
  double acc = 0.0;
  for (int r = threadIdx.x; r < g.S; r += kThreads) {
    if (g.padded) {
      const int tile = r / g.L, i = r - tile * g.L;
      const int a2 = tile % g.n2, a1 = (tile / g.n2) % g.n1, a0 = tile / (g.n2 * g.n1);
      if (!token_real(a0, a1, a2, i, g)) continue;
    }
    acc += (double)expf(lse_win[base + r] - lse_full[base + r]);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) mass[blockIdx.x] = (float)(part[0] * inv_real);
}

// One workgroup per (candidate, sequence): the fixed-order fp64 sum of the
// per-wave partial sums of the row masses (mass instance of fwd_bf16_kernel).
__global__ __launch_bounds__(kThreads) void mass_reduce_kernel(const float* __restrict__ partial,
                                                               float* __restrict__ mass,
                                                               uint32_t nblk32, double inv_real) {
  __shared__ double part[kThreads];
  const float* src = partial + (size_t)blockIdx.x * nblk32;
  double acc = 0.0;
  for (uint32_t i = threadIdx.x; i < nblk32; i += kThreads) acc += (double)src[i];
  part[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) mass[blockIdx.x] = (float)(part[0] * inv_real);
}

}  // namespace

hipError_t launch_mass_reduce(const float* partial, float* mass, const Geometry& g, int ncand,
                              int64_t BH, hipStream_t st) {
  hipLaunchKernelGGL(mass_reduce_kernel, dim3((uint32_t)(ncand * BH)), dim3(kThreads), 0, st,
                     partial, mass, (uint32_t)(g.S / 32), 1.0 / (double)g.Sr);
  return hipGetLastError();
}

hipError_t launch_mass(const float* lse_win, const float* lse_full, float* mass, const Geometry& g,
                       int64_t BH, hipStream_t st) {
  hipLaunchKernelGGL(mass_kernel, dim3((uint32_t)BH), dim3(kThreads), 0, st, lse_win, lse_full, mass,
                     g, 1.0 / (double)g.Sr);
  return hipGetLastError();
}

}  // namespace sta
