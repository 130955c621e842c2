// Calibration kernel for the benchmark: the bf16 matrix-core rate this part
// sustains from registers, with caller-chosen operand data. On MI355X the
// published dense bf16 peak assumes the full engine clock; under a sustained
// MFMA stream the clock is set by the power the matrix cores draw, and that
// draw depends on the operand bits (zeros draw little, random bf16 a lot). The
// attention kernels' operands are random bf16 data, so the random-operand
// rate measured here is the ceiling their MFMA work can approach.
#include "common.h"

namespace pa {

constexpr int PROBE_THREADS = 512;
constexpr int PROBE_OPS = 65536;   // 16-byte operand slots in the caller's buffer

// Each thread loads 8 A and 8 B operands (16 bytes each) and runs `iters`
// rounds of independent-chain MFMAs (so the matrix pipe never waits on a
// result): 32 of v_mfma_f32_32x32x16_bf16 on 4 accumulators, or the same FLOPs
// as 64 of v_mfma_f32_16x16x32_bf16 on 8 accumulators. It then stores one float
// so nothing is dead code. Per multiply-add the 16x16x32 form reads and writes
// half the accumulator bits of the 32x32x16 form and reads twice the operand
// bits.
template <int SHAPE>
__global__ void __launch_bounds__(PROBE_THREADS) mfma_probe_kernel(const u32x4* __restrict__ ops,
                                                                   float* __restrict__ sink, int iters) {
  const int t = threadIdx.x + blockIdx.x * PROBE_THREADS;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, ops[(t * 16 + 2 * i) % PROBE_OPS]);
    b[i] = __builtin_bit_cast(bf16x8, ops[(t * 16 + 2 * i + 1) % PROBE_OPS]);
  }
  float s = 0.f;
  if constexpr (SHAPE == 32) {
    f32x16 c[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + k) & 7], b[(3 * i + k) & 7], c[k], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[0][i] + c[1][i] + c[2][i] + c[3][i];
  } else {
    f32x4 c[8] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(i + k) & 7], b[(3 * i + k) & 7], c[k], 0, 0, 0);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  }
  sink[t] = s;
}

hipError_t launch_mfma_probe(const uint16_t* operands, float* sink, int grid, int iters, int shape,
                             hipStream_t stream) {
  const u32x4* ops = reinterpret_cast<const u32x4*>(operands);
  if (shape == 32)
    hipLaunchKernelGGL(mfma_probe_kernel<32>, dim3(grid), dim3(PROBE_THREADS), 0, stream, ops, sink, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3(grid), dim3(PROBE_THREADS), 0, stream, ops, sink, iters);
  return hipGetLastError();
}

}  // namespace pa
