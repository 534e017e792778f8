// Matrix-core calibration loop: the bf16 MFMA rate this GPU sustains on
// operands drawn like the attention inputs, with nothing else running.
//
// Not part of the attention method and not part of libsta: it is built as
// its own library, libsta_calib.so, for the benchmark, and gives the
// measurement a second reference next to the published dense peak.  Operand values decide how much
// power the matrix cores draw, and under the board's power limit that sets the
// clock; a loop on all-zero operands runs at the top clock, a loop on N(0, 1)
// bf16 operands may not.  Each wave keeps eight A and eight B fragments (taken
// from the caller's buffer) and cycles through them, so consecutive MFMAs see
// different operands, in four independent accumulator chains.
#include "kernels.h"
#include "mfma_common.h"

namespace sta {

namespace {

constexpr int kCalibThreads = 256;

__global__ __launch_bounds__(kCalibThreads) void calib_mfma_kernel(const u32x4* __restrict__ src,
                                                                   uint32_t src_mask, int iters,
                                                                   float* __restrict__ out) {
  const uint32_t t = blockIdx.x * kCalibThreads + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = as_bf16x8(src[(t * 16u + i) & src_mask]);
    b[i] = as_bf16x8(src[(t * 16u + 8 + i) & src_mask]);
  }
  // The four waves of a workgroup enter the loop together.  Without this
  // barrier the loads above finish at different times on different waves and
  // the loop, measured on gfx950, ran 25-40% below the rate the same loop
  // reaches when its waves start in step (zero operands: about 1700 against
  // 2470 TFLOP/s at two and three waves per SIMD); the aligned rate is the
  // one the matrix cores can sustain.
  __syncthreads();
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i & 3] = mfma32(a[i], b[(i * 3) & 7], acc[i & 3]);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i & 3] = mfma32(a[(i + 3) & 7], b[(i * 5) & 7], acc[i & 3]);
  }
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) r += acc[0][e] + acc[1][e] + acc[2][e] + acc[3][e];
  out[t] = r;
}

}  // namespace

}  // namespace sta

// int sta_calib_mfma_bf16(const void* operands, int64_t operand_bytes,
//                         int64_t iters, int64_t blocks, float* out, void* stream)
// operands: device buffer, operand_bytes a power of two >= 256, 16-byte
// aligned; blocks workgroups of 256 threads each run iters iterations of 16
// v_mfma_f32_32x32x16_bf16 per wave, i.e. blocks * 4 * iters * 16 * 32768 FLOP
// per launch.  out: device fp32 [blocks * 256], overwritten with per-thread
// sums (so the work is kept).  Asynchronous on stream (a hipStream_t, NULL =
// the null stream); returns 0, -1 for a bad argument, -5 for a misaligned
// pointer, -6 when the launch fails.
extern "C" __attribute__((visibility("default"))) int sta_calib_mfma_bf16(
    const void* operands, int64_t operand_bytes, int64_t iters, int64_t blocks, float* out,
    void* stream) {
  if (!operands || !out || iters < 1 || blocks < 1 || iters >= (1ll << 31) ||
      blocks >= (1ll << 31) / sta::kCalibThreads)
    return -1;
  const int64_t vecs = operand_bytes / 16;
  if (vecs < 16 || (vecs & (vecs - 1)) != 0 || operand_bytes % 16 != 0) return -1;
  if (((uintptr_t)operands & 15u) || ((uintptr_t)out & 15u)) return -5;
  hipLaunchKernelGGL(sta::calib_mfma_kernel, dim3((uint32_t)blocks), dim3(sta::kCalibThreads), 0,
                     (hipStream_t)stream, (const sta::u32x4*)operands, (uint32_t)(vecs - 1),
                     (int)iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
