// Forward kernel: packed branch-aware attention, bf16 MFMA, online softmax.
//
// Computes O = softmax(scale * Q K^T under the pack mask) V and the row
// log-sum-exp, visiting only the tiles the block map marks full or partial
// (a block mask that skips fully masked blocks, "DPO Preference Packing:
// Dense Masks and Sparse Execution", section "Dense and sparse execution").
// The mask is evaluated on partial tiles only, from each query's window
// [pre_lo, pre_hi) U [kv_lo, i] of visible keys.
//
// Work decomposition: a workgroup of 4 waves owns one query tile of one row
// and WGH q heads that share a kv head (grouped-query attention); each wave
// owns 32 query rows of one q head.  Workgroups are launched in the map's
// longest-list-first order, and consecutive workgroups take different head
// groups of the same query tile.  K and V tiles of 64 keys are staged in
// LDS once per workgroup with direct global-to-LDS loads (double-buffered,
// the next tile's loads in flight during this tile's math, one barrier per
// tile) and read by all of its waves.  Two workgroups share a compute unit, so one wave's
// softmax (vector ALU) overlaps the other's MFMAs.
//
// Scores are computed transposed, S^T = K Q^T (keys on MFMA rows, queries on
// MFMA columns), so each lane owns a whole query column: the softmax row max
// and sum are lane-local plus one exchange between the wave's two halves,
// and P^T in the accumulator layout is directly the B operand of
// O^T = V^T P^T.  V^T is read with LDS transpose reads.  Tiles are staged
// through buffer resources whose range ends at the row's last token, so key
// rows past it read as zeros; they only ever meet masked (partial-tile)
// scores, whose probability is exactly 0.
#include <type_traits>

#include "pba_tile.h"

namespace pba {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int D>
struct FwdCfg {
  static constexpr int NS = D / 16;  // MFMA k-steps over the head dim
  static constexpr int NE = D / 32;  // 32-wide blocks of the head dim
  static constexpr int KSTR = D + 8;   // K tile row stride (elements)
  static constexpr int VSTR = D + 8;   // V tile row stride (elements)
};

// One key tile for one wave: S^T = K Q^T (64 keys x 32 queries), online
// softmax (masked on partial tiles), O^T = alpha O^T + V^T P^T.
// Key j = k0 + 32*aa + 8*(r/4) + 4*hi + r%4 sits in register r of s[aa];
// with jb = k0 + 4*hi and o the compile-time part, j is visible to the
// lane's query iff o <= lim and (o >= lo or (unsigned)(o + pc) < plen).
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile(f32x16 (&o)[D / 32], float& m, float& l, const bf16x8 (&qop)[D / 16],
                                         const bf16* __restrict__ sk, const bf16* __restrict__ sv, float scale_log2,
                                         int lim, int lo, int pc, int plen, int lane) {
  using C = FwdCfg<D>;
  const int l32 = lane & 31, hi = lane >> 5;
  f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int st = 0; st < C::NS; ++st) {
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      const bf16x8 kop = *(const bf16x8*)(sk + prow(32 * aa + l32) * C::KSTR + 16 * st + 8 * hi);
      s[aa] = mfma32(kop, qop[st], s[aa]);
    }
  }
  sched_fence();
  float mx = kNegInf;
#pragma unroll
  for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MASK) {
        const int off = 32 * aa + 8 * (r >> 2) + (r & 3);
        const bool ok = off <= lim && (off >= lo || (unsigned)(off + pc) < (unsigned)plen);
        s[aa][r] = ok ? s[aa][r] : kNegInf;
      }
      mx = fmaxf(mx, s[aa][r]);
    }
  }
  mx = fmaxf(mx, wave_half_swap(mx)) * scale_log2;
  const float mnew = fmaxf(m, mx);
  const float mref = mnew == kNegInf ? 0.f : mnew;
  const float alpha = fast_exp2(m - mref);
  m = mnew;
  float lsum = 0.f;
  bf16x8 p[2][2];
#pragma unroll
  for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(__builtin_fmaf(s[aa][r], scale_log2, -mref));
      s[aa][r] = e;
      lsum += e;
    }
    p[aa][0] = pack8(s[aa], 0);
    p[aa][1] = pack8(s[aa], 8);
  }
  l = l * alpha + lsum;
#pragma unroll
  for (int e = 0; e < C::NE; ++e) o[e] *= alpha;
  sched_fence();
#pragma unroll
  for (int e = 0; e < C::NE; ++e) {
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = 32 * aa + 16 * u + 4 * hi;
        const bf16x8 vop = lds_tr8p(sv, C::VSTR, r0, r0 + 8, 32 * e, lane);
        o[e] = mfma32(vop, p[aa][u], o[e]);
      }
    }
  }
}

template <int D, int WGH>
__global__ void __launch_bounds__(256, 2) fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  static_assert(C::KSTR == C::VSTR, "K and V tiles share one stager");
  constexpr int T = 64 * C::KSTR;  // elements of one K or V tile
  // K/V double buffers: K(0) V(0) K(1) V(1).  The workgroup's Q block is
  // first staged in the second pair and its O block leaves through LDS.
  __shared__ __attribute__((aligned(1024))) bf16 lds[4 * T];
  constexpr int R = 32 * (4 / WGH);  // query rows of the workgroup
  using Blk = RowBlock<R, WGH * D * 2>;
  static_assert(Blk::BYTES <= 2 * T * 2 && R * Blk::LSTR <= 4 * T * 2, "Q / O block fits the LDS buffers");

  const MapView& mp = a.map;
  // The status and the work-order entry are read together (one memory
  // round trip); nothing is used before the status check.
  const int map_status = cptr(mp.status)[0];
  const int order_entry = cptr(mp.q_order)[blockIdx.x / (a.Hq / WGH)];
  // (Using the values and the list pointers here keeps the compiler from
  // sinking these loads, and the argument loads they need, below the branch:
  // each would cost a memory round trip before the first tile's loads.)
  asm volatile("" ::"s"(map_status), "s"(order_entry), "s"(mp.q2k_cnt), "s"(mp.q2k_idx));
  if (map_status != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int l32 = lane & 31, hi = lane >> 5;
  const int nhg = a.Hq / WGH;
  // b * nqt + qt, longest lists first (clamped like every map read below)
  const int item = min(max(order_entry, 0), mp.B * mp.nqt - 1);
  const int b = item / mp.nqt, qt = item % mp.nqt;
  const int h0 = (blockIdx.x % nhg) * WGH;
  const int hw = w % WGH, qb = w / WGH;  // this wave's head and 32-query block
  const int h = h0 + hw;
  const int g = h / a.G;
  const int S = a.S, Hq = a.Hq, Hkv = a.Hkv;
  const int q0 = qt * R;
  const int qi = q0 + qb * 32 + l32;  // this lane's query
  const int qrows = min(R, S - q0);
  const int qrow_bytes = Hq * D * 2;
  char* const qo_lds = (char*)lds;  // the Q block (second buffer pair) and later the O block
  char* const q_lds = qo_lds + 2 * T * 2;

  const int64_t lrow = (int64_t)b * mp.nqt + qt;
  // Counts are clamped so that even a corrupted map cannot index outside
  // the list or the tensors.
  const cint_ptr cnt = cptr(mp.q2k_cnt) + lrow * 2;
  const int n = min(max(cnt[0] + cnt[1], 0), mp.nkt);
  const int nfull = min(max(cnt[0], 0), n);
  const cint_ptr list = cptr(mp.q2k_idx) + lrow * mp.nkt;

  const int kvstride = Hkv * D;
  const bf16* kb = a.k + ((int64_t)b * S * Hkv + g) * D;
  const bf16* vb = a.v + ((int64_t)b * S * Hkv + g) * D;
  const Stager<D, C::KSTR> kst(tid, kvstride);
  auto sK = [&](int buf) { return lds + (2 * buf) * T; };
  auto sV = [&](int buf) { return lds + (2 * buf + 1) * T; };

  // Prologue: the Q block and the first K/V tile, all as direct loads.
  Blk::template load<4>(q_lds, a.q + ((int64_t)b * S + q0) * Hq * D + (int64_t)h0 * D, qrows, qrow_bytes, w, lane);
  const int first = list[0];  // valid memory even for an empty list
  asm volatile("" ::"s"(first), "s"(n));
  if (n > 0) {
    const int k0 = min(max(first, 0), mp.nkt - 1) * 64;
    kst.stage(sK(0), kb + (int64_t)k0 * kvstride, S - k0);
    kst.stage(sV(0), vb + (int64_t)k0 * kvstride, S - k0);
  }
  int wlo, wplo, wphi;
  {
    const int4 wv = reinterpret_cast<const int4*>(mp.tok_win)[(int64_t)b * S + min(qi, S - 1)];
    wlo = qi < S ? wv.x : qi + 1;
    wplo = qi < S ? wv.y : 0;
    wphi = qi < S ? wv.z : 0;
  }
  wait_vmem();
  __syncthreads();
  // Q^T as the B operand: lane holds query qi, head dims 16*st + 8*hi + 0..7.
  bf16x8 qop[C::NS];
  {
    const char* qr = q_lds + (qb * 32 + l32) * Blk::LSTR + hw * D * 2 + 16 * hi;
#pragma unroll
    for (int st = 0; st < C::NS; ++st) qop[st] = *(const bf16x8*)(qr + 32 * st);
  }
  __syncthreads();  // the second buffer pair is free again

  float m = kNegInf, l = 0.f;
  f32x16 o[C::NE];
#pragma unroll
  for (int e = 0; e < C::NE; ++e) o[e] = f32x16{};

  // One visit: start the next tile's loads into the other buffer (last read
  // in the previous visit, which every wave has left), then this tile's math.
  auto visit = [&](int j, auto masked) {
    const int kt = min(max(list[j], 0), mp.nkt - 1);
    const int buf = j & 1;
    if (j + 1 < n) {
      const int k0 = min(max(list[j + 1], 0), mp.nkt - 1) * 64;
      kst.stage(sK(buf ^ 1), kb + (int64_t)k0 * kvstride, S - k0);
      kst.stage(sV(buf ^ 1), vb + (int64_t)k0 * kvstride, S - k0);
    }
    if constexpr (decltype(masked)::value) {
      const int jb = kt * 64 + 4 * hi;
      fwd_tile<D, true>(o, m, l, qop, sK(buf), sV(buf), a.scale_log2, qi - jb, wlo - jb, jb - wplo, wphi - wplo, lane);
    } else {
      fwd_tile<D, false>(o, m, l, qop, sK(buf), sV(buf), a.scale_log2, 0, 0, 0, 0, lane);
    }
    wait_vmem();
    __syncthreads();
  };
  // Full tiles come first in the list, then partial ones.  Two loops rather
  // than a branch in one keep each loop's accumulators in place (a merge of
  // two paths inside one loop body costs a copy of every accumulator).
  int j = 0;
  for (; j < nfull; ++j) visit(j, std::false_type{});
  for (; j < n; ++j) visit(j, std::true_type{});

  // Epilogue: normalise; O (bf16) goes through LDS (free after the last
  // barrier) so that its rows leave as whole contiguous segments; LSE in
  // natural log.
  const float lt = l + wave_half_swap(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  {
    char* orow = qo_lds + (qb * 32 + l32) * Blk::LSTR + hw * D * 2 + 8 * hi;
#pragma unroll
    for (int e = 0; e < C::NE; ++e) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (bf16)(o[e][4 * rg + t] * inv);
        *(bf16x4*)(orow + 2 * (32 * e + 8 * rg)) = v;
      }
    }
  }
  if (qi < S && hi == 0) a.lse[((int64_t)b * Hq + h) * S + qi] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
  __syncthreads();
  Blk::template store<256>(a.o + ((int64_t)b * S + q0) * Hq * D + (int64_t)h0 * D, qo_lds, qrows, qrow_bytes, tid);
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, int wgh, unsigned nblk, hipStream_t stream) {
  switch (wgh) {
    case 4:
      hipLaunchKernelGGL((fwd_kernel<D, 4>), dim3(nblk), dim3(256), 0, stream, a);
      break;
    case 2:
      hipLaunchKernelGGL((fwd_kernel<D, 2>), dim3(nblk), dim3(256), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((fwd_kernel<D, 1>), dim3(nblk), dim3(256), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int fwd_wg_heads(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1); }

hipError_t launch_fwd(const FwdArgs& a, int D, int B, hipStream_t stream) {
  const int wgh = fwd_wg_heads(a.G);
  const unsigned nblk = (unsigned)((int64_t)B * a.map.nqt * (a.Hq / wgh));
  return D == 128 ? launch_fwd_d<128>(a, wgh, nblk, stream) : launch_fwd_d<64>(a, wgh, nblk, stream);
}

}  // namespace pba
