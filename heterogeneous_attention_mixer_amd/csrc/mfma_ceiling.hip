// mfma_ceiling.hip -- measurement aid: the bf16 matrix-core rate this GPU sustains under its
// power cap when nothing but matrix instructions runs. The prefill kernels are rated against
// it beside the data-sheet peak (which assumes the 2.4 GHz clock).
//
// Every wave keeps four independent accumulator chains of v_mfma_f32_32x32x16_bf16 in
// flight (an MFMA that accumulates into the result of the one just before it waits for that
// result), on operands that change from one instruction to the next: the power drawn by the
// matrix cores depends on how many operand bits toggle, so the operands are the caller's
// seeded random bf16 fragments rather than constants.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace mixer {

namespace {

// Fragment set s (8 fragments of 64 lanes x 8 bf16): fragments 0-3 are A operands (lane l
// holds row l % 32, k = 8 * (l / 32) + [0, 8) of a 32 x 16 matrix), fragments 4-7 are B
// operands (lane l holds column l % 32, the same k). Wave w uses set w % nsets. After `iters`
// instructions per chain (a multiple of 4), chain c holds
//   (iters / 4) * sum_{u=0..3} A[(u + c) % 4] * B[(u + 2c) % 4],
// written as sink[((w * 4 + c) * 16 + r) * 64 + lane] for accumulator element r.
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
mfma_ceiling_kernel(const bf16x8* __restrict__ frags, int nsets, float* __restrict__ sink,
                    int iters) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bf16x8* f = frags + (size_t)(w % nsets) * 8 * 64;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = f[i * 64 + lane];
    b[i] = f[(4 + i) * 64 + lane];
  }
  floatx16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int t = 0; t < iters; t += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32(a[(u + c) & 3], b[(u + 2 * c) & 3], acc[c]);
  }
  float* s = sink + (size_t)w * 4 * 16 * 64;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[(c * 16 + r) * 64 + lane] = acc[c][r];
}

}  // namespace

hipError_t launch_mfma_ceiling(const void* frags, int nsets, float* sink, int blocks, int iters,
                               hipStream_t stream) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const bf16x8*>(frags), nsets, sink, iters);
  return hipGetLastError();
}

}  // namespace mixer
