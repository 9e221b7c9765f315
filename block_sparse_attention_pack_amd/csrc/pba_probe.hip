// Measurement helper, not part of the attention path: a fixed loop of
// v_mfma_f32_32x32x16_bf16 with four independent accumulators per wave,
// which sets the sustained bf16 MFMA rate of the device (clock under load
// included) against which the attention kernels can be compared.
#include "pba_tile.h"

namespace pba {
namespace {

__global__ void __launch_bounds__(256) mfma_probe(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    a[t] = (bf16)(float)((lane + t) & 7);
    b[t] = (bf16)(float)((lane * 3 + t) & 7);
  }
  f32x16 c[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = mfma32(a, b, c[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += c[i][0] + c[i][15];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int n_blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe, dim3(n_blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace pba
