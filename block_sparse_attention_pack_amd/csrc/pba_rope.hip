// Rotary embedding at the packed, branch-aligned position ids ("DPO
// Preference Packing: Dense Masks and Sparse Execution", section "Layout
// requirements": each response keeps the positions of its own
// [prompt | response] sequence).  The position of token s comes from the
// block map: for a pack token, the length of the earlier visible run (the
// prompt, for a response token) plus the offset of s in its own run; pad
// tokens get position 0 (the identity).  Rotate-half pairing: head dim i
// pairs with i + D/2, frequency base^(-2i/D):
//
//   y[i]       = x[i] cos(a) - x[i + D/2] sin(a),   a = pos * f_i
//   y[i + D/2] = x[i] sin(a) + x[i + D/2] cos(a)
//
// and the inverse (for gradients) rotates by -a.
//
// One wave per token: lane l owns 4 consecutive pairs (8-byte loads of each
// half) of every (64 / (D/8))-th head, computes their 4 sin/cos once and
// walks the heads.  Bound by HBM: 2 * H * D * 2 bytes per token.
#include "pba_next.h"
#include "pba_tile.h"

namespace pba {
namespace {

constexpr int kRopeWaves = 4;

template <int D>
__global__ void __launch_bounds__(64 * kRopeWaves) rope_apply(RopeArgs a) {
  if (a.status[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kRopeWaves + (threadIdx.x >> 6);  // token b * S + s
  if (t >= a.ntok) return;
  constexpr int NG = D / 8;         // groups of 4 pairs per head
  constexpr int HP = 64 / NG;       // heads per pass of the wave
  const int gi = lane % NG, ho = lane / NG;
  const int s = (int)(t % a.S);
  const int4 w = reinterpret_cast<const int4*>(a.tok_win)[t];
  const bool pad = a.tok_pack[t] < 0;
  const int pos = pad ? 0 : (w.z - w.y) + (s - w.x);
  float c[4], sn[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * gi + j;
    const float f = exp2f(-(float)(2 * i) / (float)D * a.log2_base);
    const float ang = (float)pos * f * a.sign;
    sincosf(ang, &sn[j], &c[j]);
  }
  const bf16* x = a.x + t * a.H * D;
  bf16* y = a.y + t * a.H * D;
  for (int h = ho; h < a.H; h += HP) {
    const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(x + h * D + 4 * gi);
    const bf16x4 x2 = *reinterpret_cast<const bf16x4*>(x + h * D + D / 2 + 4 * gi);
    bf16x4 y1, y2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float u = (float)x1[j], v = (float)x2[j];
      y1[j] = (bf16)(u * c[j] - v * sn[j]);
      y2[j] = (bf16)(u * sn[j] + v * c[j]);
    }
    *reinterpret_cast<bf16x4*>(y + h * D + 4 * gi) = y1;
    *reinterpret_cast<bf16x4*>(y + h * D + D / 2 + 4 * gi) = y2;
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, int D, hipStream_t stream) {
  const unsigned nblk = (unsigned)((a.ntok + kRopeWaves - 1) / kRopeWaves);
  if (D == 128) hipLaunchKernelGGL(rope_apply<128>, dim3(nblk), dim3(64 * kRopeWaves), 0, stream, a);
  else hipLaunchKernelGGL(rope_apply<64>, dim3(nblk), dim3(64 * kRopeWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pba
