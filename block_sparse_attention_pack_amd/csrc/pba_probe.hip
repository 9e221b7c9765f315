// Measurement helpers, not part of the attention path: fixed loops that set
// the sustained rates of the device's units (clock under load included)
// against which the attention kernels can be compared.
//   mfma_probe  v_mfma_f32_32x32x16_bf16, four independent accumulators per
//               wave
//   lds_probe   16-byte LDS reads, lane-contiguous 1 KB per wave (no bank
//               conflicts), 16 per iteration in four independent chains
//   valu_probe  16 independent chains per lane of fp32 FMA, or of exp2
//               (v_exp_f32) followed by one multiply
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

// 512 threads, a 64 KB LDS array; every read stays inside it.
__global__ void __launch_bounds__(512) lds_probe(float* out, int iters) {
  __shared__ f32x4 buf[4096];
  const int tid = threadIdx.x;
  for (int i = tid; i < 4096; i += 512) buf[i] = f32x4{(float)i, 1.f, 2.f, 3.f};
  __syncthreads();
  f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u & 3] += buf[(tid + 64 * u + it) & 4095];
  }
  const f32x4 t = acc[0] + acc[1] + acc[2] + acc[3];
  out[(size_t)blockIdx.x * 512 + tid] = t[0] + t[1] + t[2] + t[3];
}

template <bool EXP>
__global__ void __launch_bounds__(256) valu_probe(float* out, int iters) {
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = (float)(threadIdx.x + j) * 1e-6f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = EXP ? __builtin_amdgcn_exp2f(v[j]) * -0.5f : __builtin_fmaf(v[j], 0.999f, 1e-7f);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += v[j];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_lds_probe(float* out, int n_blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(lds_probe, dim3(n_blocks), dim3(512), 0, stream, out, iters);
  return hipGetLastError();
}

hipError_t launch_valu_probe(float* out, int n_blocks, int iters, int exp, hipStream_t stream) {
  if (exp) hipLaunchKernelGGL(valu_probe<true>, dim3(n_blocks), dim3(256), 0, stream, out, iters);
  else hipLaunchKernelGGL(valu_probe<false>, dim3(n_blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int n_blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe, dim3(n_blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace pba
