// Forward kernel: packed branch-aware attention, bf16 MFMA, online softmax.
//
// Computes O = softmax(scale * Q K^T under the pack mask) V and the row
// log-sum-exp, visiting only the tiles the block map marks full or partial
// (a block mask skipping fully masked blocks, "DPO Preference Packing: Dense
// Masks and Sparse Execution", section "Dense and sparse execution").  The
// mask is evaluated on partial tiles only, from each query's window
// [pre_lo, pre_hi) U [kv_lo, i] of visible keys.
//
// Work decomposition: a workgroup of 4 waves owns one query tile of one row
// and WGH q heads that share a kv head (grouped-query attention); each wave
// owns 64 query rows of one q head.  K and V tiles of 64 keys are staged in
// LDS once per workgroup and read by all its waves, double-buffered with a
// register prefetch of the next tile from HBM.
//
// Scores are computed transposed, S^T = K Q^T (keys on MFMA rows, queries on
// MFMA columns), so each lane owns whole query columns: the softmax row max
// and sum are lane-local plus one swap between the wave's two halves, and
// P^T in the accumulator layout is directly the B operand of O^T = V^T P^T.
// V^T is read with LDS transpose reads from the row-major V tile.
#include "pba_tile.h"

namespace pba {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int D, int WGH>
__global__ void __launch_bounds__(256, 1) fwd_kernel(FwdArgs a) {
  constexpr int NS = D / 16;         // MFMA k-steps over the head dim
  constexpr int NE = D / 32;         // 32-wide blocks of the head dim
  constexpr int KSTR = D + 8;        // K tile row stride (elements)
  constexpr int VSTR = D + 16;       // V tile row stride (elements)
  constexpr int CH = 64 * D / 8 / 256;  // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 sK[2][64 * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][64 * VSTR];

  const MapView& mp = a.map;
  if (mp.status[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qt = blockIdx.x, b = blockIdx.z;
  const int h = blockIdx.y * WGH + (w % WGH);
  const int g = h / a.G;
  const int S = a.S, Hq = a.Hq, Hkv = a.Hkv;
  const int q0 = qt * (64 * (4 / WGH)) + (w / WGH) * 64;

  // Q^T as the B operand: lane holds query column q0 + 32c + l32, head dims
  // 16*st + 8*hi + 0..7.
  bf16x8 qop[2][NS];
  int wlo[2], wplo[2], wphi[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int qi = q0 + 32 * c + l32;
    if (qi < S) {
      const bf16* qrow = a.q + (((int64_t)b * S + qi) * Hq + h) * D + 8 * hi;
#pragma unroll
      for (int st = 0; st < NS; ++st) qop[c][st] = *(const bf16x8*)(qrow + 16 * st);
      const int4 wv = reinterpret_cast<const int4*>(mp.tok_win)[(int64_t)b * S + qi];
      wlo[c] = wv.x; wplo[c] = wv.y; wphi[c] = wv.z;
    } else {
#pragma unroll
      for (int st = 0; st < NS; ++st) qop[c][st] = bf16x8{};
      wlo[c] = qi + 1; wplo[c] = 0; wphi[c] = 0;
    }
  }

  const int64_t lrow = (int64_t)b * mp.nqt + qt;
  // Counts are clamped so that even a corrupted map cannot index outside
  // the list or the tensors.
  const int ntot = min(max(mp.q2k_cnt[lrow * 2] + mp.q2k_cnt[lrow * 2 + 1], 0), mp.nkt);
  const int nfull = min(max(mp.q2k_cnt[lrow * 2], 0), ntot);
  const int32_t* list = mp.q2k_idx + lrow * mp.nkt;

  float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
  f32x16 o[NE][2];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e][0] = o[e][1] = f32x16{};

  uint4 rk[CH], rv[CH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), c8 = c % (D / 8);
      const int kj = kt * 64 + r;
      if ((unsigned)kj < (unsigned)S) {
        const int64_t off = (((int64_t)b * S + kj) * Hkv + g) * D + 8 * c8;
        rk[i] = *(const uint4*)(a.k + off);
        rv[i] = *(const uint4*)(a.v + off);
      } else {
        rk[i] = rv[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), c8 = c % (D / 8);
      *(uint4*)&sK[buf][r * KSTR + 8 * c8] = rk[i];
      *(uint4*)&sV[buf][r * VSTR + 8 * c8] = rv[i];
    }
  };

  if (ntot > 0) {
    gload(list[0]);
    sstore(0);
  }
  __syncthreads();

  for (int it = 0; it < ntot; ++it) {
    const int kt = list[it];
    const int buf = it & 1;
    if (it + 1 < ntot) gload(list[it + 1]);

    // S^T = K Q^T: rows = keys 32*aa + ..., columns = this wave's queries.
    f32x16 s[2][2];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) s[aa][0] = s[aa][1] = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
        const bf16x8 kop = *(const bf16x8*)&sK[buf][(32 * aa + l32) * KSTR + 16 * st + 8 * hi];
        s[aa][0] = mfma32(kop, qop[0][st], s[aa][0]);
        s[aa][1] = mfma32(kop, qop[1][st], s[aa][1]);
      }
    }

    const bool partial = it >= nfull;
    const int k0 = kt * 64;
    bf16x8 pop[2][2][2];  // [query block][key block][k-step half]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qi = q0 + 32 * c + l32;
      float mx = kNegInf;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[aa][c][r] * a.scale_log2;
          if (partial) {
            const int j = k0 + 32 * aa + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = j <= qi && (j >= wlo[c] || (j >= wplo[c] && j < wphi[c]));
            x = ok ? x : kNegInf;
          }
          s[aa][c][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, wave_half_swap(mx));
      const float mnew = fmaxf(m[c], mx);
      const float mref = mnew == kNegInf ? 0.f : mnew;
      const float alpha = fast_exp2(m[c] - mref);
      m[c] = mnew;
      float lsum = 0.f;
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(s[aa][c][r] - mref);
          s[aa][c][r] = p;
          lsum += p;
        }
        pop[c][aa][0] = pack8(s[aa][c], 0);
        pop[c][aa][1] = pack8(s[aa][c], 8);
      }
      l[c] = l[c] * alpha + lsum;
#pragma unroll
      for (int e = 0; e < NE; ++e) o[e][c] *= alpha;
    }

    // O^T += V^T P^T: A = V^T (transpose-read, key order matching P^T's
    // accumulator layout), B = P^T.
#pragma unroll
    for (int e = 0; e < NE; ++e) {
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 32 * aa + 16 * u + 4 * hi;
          const bf16x8 vop = lds_tr8(sV[buf], VSTR, r0, r0 + 8, 32 * e, lane);
          o[e][0] = mfma32(vop, pop[0][aa][u], o[e][0]);
          o[e][1] = mfma32(vop, pop[1][aa][u], o[e][1]);
        }
      }
    }

    if (it + 1 < ntot) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: normalise, write O (bf16) and LSE (natural log).
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float lt = l[c] + wave_half_swap(l[c]);
    const int qi = q0 + 32 * c + l32;
    if (qi < S) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      bf16* orow = a.o + (((int64_t)b * S + qi) * Hq + h) * D + 4 * hi;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (bf16)(o[e][c][4 * rg + t] * inv);
          *(bf16x4*)(orow + 32 * e + 8 * rg) = v;
        }
      }
      if (hi == 0)
        a.lse[((int64_t)b * Hq + h) * S + qi] = lt > 0.f ? (m[c] + __log2f(lt)) * kLn2 : kNegInf;
    }
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, int B, hipStream_t stream) {
  const int wgh = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0 ? 2 : 1);
  dim3 grid(a.map.nqt, a.Hq / wgh, B);
  if (wgh == 4) fwd_kernel<D, 4><<<grid, 256, 0, stream>>>(a);
  else if (wgh == 2) fwd_kernel<D, 2><<<grid, 256, 0, stream>>>(a);
  else fwd_kernel<D, 1><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

int fwd_wg_heads(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1); }

hipError_t launch_fwd(const FwdArgs& a, int D, int B, hipStream_t stream) {
  return D == 128 ? launch_fwd_d<128>(a, B, stream) : launch_fwd_d<64>(a, B, stream);
}

}  // namespace pba
