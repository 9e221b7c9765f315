// Device helpers for the attention kernels: MFMA wrappers, LDS transpose
// reads, bf16 packing.  Lane layouts (wave64, verified on gfx950):
//   v_mfma_f32_32x32x16_bf16:  A[i][k]: lane l holds i = l%32, k = 8*(l/32)+0..7
//                              B[k][j]: lane l holds j = l%32, k = 8*(l/32)+0..7
//                              C[i][j]: lane l, register r holds
//                                       j = l%32, i = 8*(r/4) + 4*(l/32) + r%4
//   ds_read_b64_tr_b16: in each group of 16 lanes, source lane s addresses 4
//     consecutive 16-bit elements; destination lane i receives element i%4
//     of source lanes i/4, 4+i/4, 8+i/4, 12+i/4.  If source lane s points at
//     M[r0 + s/4][c0 + 4*(s%4)] of a row-major matrix M, lane i receives
//     M[r0 + t][c0 + i] for t = 0..3: a 4 x 16 block read column-wise.
#pragma once
#include "pba_internal.h"

namespace pba {

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PBA_LDS i16x4*)((PBA_LDS char*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// 8 values for a 32x32x16 operand whose k index runs down the rows of a
// row-major LDS matrix M (row stride `stride` elements):
// lane l gets M[rows(t)][col0 + 16*((l/16)%2) + l%16] where rows(t) = r0 + t
// for t < 4 and r1 + t - 4 for t >= 4 (r0, r1 already include the lane's
// 4*(l/32) offset chosen by the caller).
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* M, int stride, int r0, int r1, int col0, int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int col = col0 + 16 * (G & 1) + 4 * (s & 3);
  const bf16x4 lo = lds_tr4(M + (r0 + (s >> 2)) * stride + col);
  const bf16x4 hi = lds_tr4(M + (r1 + (s >> 2)) * stride + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (bf16)x[base + t];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_half_swap(float x) { return __shfl_xor(x, 32); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pba
