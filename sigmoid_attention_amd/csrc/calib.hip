// Measurement aid: the bf16 MFMA rate and the shader clock this GPU sustains, the
// reference against which the attention kernels' throughput is also reported. Every wave
// runs a loop of v_mfma_f32_32x32x16_bf16 on four independent accumulators (no
// dependency stalls, no memory traffic in the loop). Thread 0 of each workgroup records
// the workgroup's elapsed shader-clock cycles (s_memtime) and 100 MHz ticks
// (s_memrealtime), from which the host forms the clock; each thread writes one float
// so that the products stay live.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace sa {

constexpr int kCalibMfmaPerIter = 16;   // four accumulators x four k-steps

__global__ __launch_bounds__(256) void mfma_calib_kernel(float* sink, int64_t* clk, int iters) {
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  const int tid = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(0.001f * ((tid + i) & 15));
    b[i] = (bf16)(0.002f * ((tid * 3 + i) & 15));
  }
  f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c0 = mfma(a, b, c0);
      c1 = mfma(b, a, c1);
      c2 = mfma(a, a, c2);
      c3 = mfma(b, b, c3);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  sink[tid] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
    clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

int calib_mfma_per_iter() { return kCalibMfmaPerIter; }

hipError_t launch_mfma_calib(float* sink, int64_t* clk, int nblocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_calib_kernel, dim3(nblocks), dim3(256), 0, st, sink, clk, iters);
  return hipGetLastError();
}

}  // namespace sa
