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
// groups of the same query tile.  The Q block and the K and V tiles of 64
// keys are staged in LDS once per workgroup with direct global-to-LDS loads
// and read by all of its waves.  The key tiles are software-pipelined: a
// step runs P V of tile j-1, the softmax of tile j and the scores of tile
// j+1 (hand-scheduled so that MFMAs and the softmax's vector work alternate
// within a wave), with K loaded two steps ahead and V one step ahead and one
// barrier per step.  Two workgroups share a compute unit, so each SIMD also
// interleaves two waves.
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

// Running-max update with a lazy reference (log2 domain): the reference m
// moves only when the tile max exceeds it by more than kLazy, so most
// tiles leave the accumulators as they are (alpha = 1).  Unnormalised
// probabilities then stay below 2^kLazy, far inside the range of the fp32
// accumulators and of bf16.  The result does not depend on the reference
// (O and LSE are normalised by the same running sum), up to rounding.
constexpr float kLazy = 8.f;
__device__ __forceinline__ float lazy_reference(float& m, float mx, float& alpha) {
  const bool move = mx > m + kLazy;  // any finite mx moves m = -inf
  alpha = move ? fast_exp2(m - mx) : 1.f;
  m = move ? mx : m;
  return m == kNegInf ? 0.f : m;
}

// O^T *= alpha, skipped when every lane's alpha is 1 (wave-uniform branch).
template <int D>
__device__ __forceinline__ void rescale(f32x16 (&o)[D / 32], float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int e = 0; e < D / 32; ++e) o[e] *= alpha;
  }
}

template <int D>
struct FwdCfg {
  static constexpr int NS = D / 16;  // MFMA k-steps over the head dim
  static constexpr int NE = D / 32;  // 32-wide blocks of the head dim
  static constexpr int KSTR = D + 8;   // K tile row stride (elements)
  static constexpr int VSTR = D + 8;   // V tile row stride (elements)
};

// The three parts of a key tile for one wave (64 keys x 32 queries).  The
// kernel runs them software-pipelined: in one step, the scores of tile j+1,
// the softmax of tile j and the P V product of tile j-1 are independent, so
// MFMAs of one part overlap the vector ALU work of another within the wave.

// S^T = K Q^T.  Key k0 + 32*aa + 8*(r/4) + 4*hi + r%4 sits in register r of
// s[aa]; the lane's query column is lane % 32.
template <int D>
__device__ __forceinline__ void fwd_scores(f32x16 (&s)[2], const bf16x8 (&qop)[D / 16], const bf16* __restrict__ sk,
                                           int lane) {
  using C = FwdCfg<D>;
  const int l32 = lane & 31, hi = lane >> 5;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int st = 0; st < C::NS; ++st) {
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      const bf16x8 kop = *(const bf16x8*)(sk + prow(32 * aa + l32) * C::KSTR + 16 * st + 8 * hi);
      s[aa] = mfma32(kop, qop[st], s[aa]);
    }
  }
}

// Online softmax of one tile (masked on partial tiles): updates the running
// reference m (log2 domain) and sum l, returns the rescale factor alpha of the
// accumulators and P^T packed as bf16 B operands.  On partial tiles, key
// jb + o (jb = k0 + 4*hi, o the compile-time part of its register's key
// offset) is visible to the lane's query iff bit o of km is set.
template <bool MASK>
__device__ __forceinline__ void fwd_softmax(f32x16 (&s)[2], float& m, float& l, float& alpha, bf16x8 (&p)[2][2],
                                            float scale_log2, KeyMask km) {
  float mx = kNegInf;
#pragma unroll
  for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (MASK) s[aa][r] = keep_or_ninf(mask_bit(aa ? km.hi : km.lo, 8 * (r >> 2) + (r & 3)), s[aa][r]);
      mx = fmaxf(mx, s[aa][r]);
    }
  }
  mx = fmaxf(mx, wave_half_swap(mx)) * scale_log2;
  const float mref = lazy_reference(m, mx, alpha);
  float lsum = 0.f;
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
}

// One full pipeline step for one wave, hand-scheduled: the MFMAs of P V
// for the previous tile (after the rescale by its alpha) and of the scores
// for the next tile, each followed by a slice of the current tile's softmax
// (mask and max while P V runs, exp and sum while the scores run), with
// every MFMA's LDS operand read two MFMAs ahead.  On return s holds the
// next tile's scores and p / alpha the current tile's P and rescale.
template <int D, bool MASK>
__device__ __forceinline__ void fwd_step(f32x16 (&o)[D / 32], bf16x8 (&p)[2][2], float& alpha, float& m, float& l,
                                         f32x16 (&s)[2], const bf16x8 (&qop)[D / 16], const bf16* __restrict__ sk,
                                         const bf16* __restrict__ sv, float scale_log2, KeyMask km, int lane) {
  using C = FwdCfg<D>;
  constexpr int NPV = C::NE * 4, NQK = C::NS * 2, N = NPV + NQK;
  constexpr int NEXP = NQK - 2;  // score slices of the exp phase (the max arrives after two MFMAs)
  const int l32 = lane & 31, hi = lane >> 5;
  auto operand = [&](int i) __attribute__((always_inline)) -> bf16x8 {
    if (i < NPV) {
      const int e = i >> 2, aa = (i >> 1) & 1, u = i & 1;
      const int r0 = 32 * aa + 16 * u + 4 * hi;
      return lds_tr8p(sv, C::VSTR, r0, r0 + 8, 32 * e, lane);
    }
    const int k = i - NPV, st = k >> 1, aa = k & 1;
    return *(const bf16x8*)(sk + prow(32 * aa + l32) * C::KSTR + 16 * st + 8 * hi);
  };
  rescale<D>(o, alpha);
  bf16x8 ops[3];
  ops[0] = operand(0);
  ops[1] = operand(1);
  f32x16 sn[2] = {f32x16{}, f32x16{}};
  float mx = kNegInf, mref = 0.f, lsum = 0.f;
  sched_fence();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 2 < N) ops[(i + 2) % 3] = operand(i + 2);
    if (i < NPV) {
      const int e = i >> 2, aa = (i >> 1) & 1, u = i & 1;
      o[e] = mfma32(ops[i % 3], p[aa][u], o[e]);
      // Mask and max of scores [32 i / NPV, 32 (i + 1) / NPV).
#pragma unroll
      for (int x = 32 * i / NPV; x < 32 * (i + 1) / NPV; ++x) {
        const int sa = x >> 4, r = x & 15;
        if (MASK) s[sa][r] = keep_or_ninf(mask_bit(sa ? km.hi : km.lo, 8 * (r >> 2) + (r & 3)), s[sa][r]);
        mx = fmaxf(mx, s[sa][r]);
      }
    } else {
      const int k = i - NPV, st = k >> 1, aa = k & 1;
      sn[aa] = mfma32(ops[i % 3], qop[st], sn[aa]);
      if (k == 1) {
        mref = lazy_reference(m, half_max(mx) * scale_log2, alpha);
      }
      if (k >= 2) {
        const int c = k - 2;
#pragma unroll
        for (int x = 32 * c / NEXP; x < 32 * (c + 1) / NEXP; ++x) {
          const int sa = x >> 4, r = x & 15;
          const float ev = fast_exp2(__builtin_fmaf(s[sa][r], scale_log2, -mref));
          s[sa][r] = ev;
          lsum += ev;
        }
      }
    }
    sched_fence();
  }
  p[0][0] = pack8(s[0], 0);
  p[0][1] = pack8(s[0], 8);
  p[1][0] = pack8(s[1], 0);
  p[1][1] = pack8(s[1], 8);
  l = l * alpha + lsum;
  s[0] = sn[0];
  s[1] = sn[1];
}

// O^T = alpha O^T + V^T P^T, V^T read with LDS transpose reads.
template <int D>
__device__ __forceinline__ void fwd_pv(f32x16 (&o)[D / 32], const bf16x8 (&p)[2][2], float alpha,
                                       const bf16* __restrict__ sv, int lane) {
  using C = FwdCfg<D>;
  const int hi = lane >> 5;
  rescale<D>(o, alpha);
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

template <int D, int WGH, bool ROPE>
__global__ void __launch_bounds__(256, 2) fwd_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  static_assert(C::KSTR == C::VSTR, "K and V tiles share one stager");
  constexpr int T = 64 * C::KSTR;  // elements of one K or V tile
  // K(0) K(1) V(0) V(1) double buffers.  The workgroup's Q block is first
  // staged in the V pair and its O block leaves through LDS.
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
  char* const qo_lds = (char*)lds;  // the O block at the end
  char* const q_lds = qo_lds + 2 * T * 2;  // the Q block at the start (the V pair)

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
  auto sK = [&](int t) { return lds + (t & 1) * T; };        // K of visit t
  auto sV = [&](int t) { return lds + (2 + (t & 1)) * T; };  // V of visit t
  auto key0 = [&](int t) { return min(max(list[t], 0), mp.nkt - 1) * 64; };

  // Prologue: the Q block and the first two K tiles, all as direct loads.  A
  // query tile that visits no key tile holds only pad rows (O = 0, LSE =
  // -inf): its Q block is read only when the rotated Q is to be written.
  if (n > 0 || (ROPE && a.q_rot))
    Blk::template load<4>(q_lds, a.q + ((int64_t)b * S + q0) * Hq * D + (int64_t)h0 * D, qrows, qrow_bytes, w, lane);
  const int first = list[0];  // valid memory even for an empty list
  asm volatile("" ::"s"(first), "s"(n));
  if (n > 0) {
    const int k0 = min(max(first, 0), mp.nkt - 1) * 64;
    kst.stage(sK(0), kb + (int64_t)k0 * kvstride, S - k0);
  }
  if (n > 1) kst.stage(sK(1), kb + (int64_t)key0(1) * kvstride, S - key0(1));
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
  if constexpr (ROPE) {
    // Rotary embedding of Q at the query's packed position (pad: 0, the
    // identity; a pad query's window starts after itself): head dim d pairs
    // with d + D/2, i.e. qop[st] with qop[st + NS/2] in the same lane.
    const int pos = wlo > qi ? 0 : (wphi - wplo) + (qi - wlo);
    const float pr = (float)pos * 0.15915494309189535f;  // revolutions per unit frequency
#pragma unroll
    for (int st = 0; st < C::NS / 2; ++st) {
      bf16x8 u = qop[st], v = qop[st + C::NS / 2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 16 * st + 8 * hi + j;
        float rev = pr * exp2f(-(float)(2 * d) / (float)D * a.rope_log2_base);
        rev -= floorf(rev);
        const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
        const float x1 = (float)u[j], x2 = (float)v[j];
        u[j] = (bf16)(x1 * cs - x2 * sn);
        v[j] = (bf16)(x1 * sn + x2 * cs);
      }
      qop[st] = u;
      qop[st + C::NS / 2] = v;
    }
    if (a.q_rot) {
      // The rotated block leaves through LDS as whole rows for the backward.
      char* qw = q_lds + (qb * 32 + l32) * Blk::LSTR + hw * D * 2 + 16 * hi;
#pragma unroll
      for (int st = 0; st < C::NS; ++st) *(bf16x8*)(qw + 32 * st) = qop[st];
      __syncthreads();
      Blk::template store<256>(a.q_rot + ((int64_t)b * S + q0) * Hq * D + (int64_t)h0 * D, q_lds, qrows, qrow_bytes,
                               tid);
    }
  }

  float m = kNegInf, l = 0.f, alpha = 1.f;
  f32x16 o[C::NE];
#pragma unroll
  for (int e = 0; e < C::NE; ++e) o[e] = f32x16{};
  f32x16 s[2];
  bf16x8 p[2][2];
  if (n > 0) fwd_scores<D>(s, qop, sK(0), lane);
  __syncthreads();  // the Q block and K(0) have been read by every wave

  // Step j (software pipeline): loads of V(j) and K(j+2) go into buffers
  // last read in step j-1; then P V of tile j-1, the scores of tile j+1
  // (K(j+1) was loaded in step j-1) and the softmax of tile j, which are
  // independent of one another.  One barrier per step.
  auto step = [&](int j, auto masked, auto has_prev, auto has_next) {
    kst.stage(sV(j), vb + (int64_t)key0(j) * kvstride, S - key0(j));
    if (j + 2 < n) kst.stage(sK(j), kb + (int64_t)key0(j + 2) * kvstride, S - key0(j + 2));
    const int jb = key0(j) + 4 * hi;
    constexpr bool MASKED = decltype(masked)::value;
    const KeyMask km = MASKED ? key_mask(qi - jb, wlo - jb, jb - wplo, wphi - wplo) : KeyMask{0u, 0u};
    if constexpr (decltype(has_prev)::value && decltype(has_next)::value) {
      fwd_step<D, MASKED>(o, p, alpha, m, l, s, qop, sK(j + 1), sV(j - 1), a.scale_log2, km, lane);
    } else {
      if constexpr (decltype(has_prev)::value) fwd_pv<D>(o, p, alpha, sV(j - 1), lane);
      f32x16 sn[2];
      if constexpr (decltype(has_next)::value) fwd_scores<D>(sn, qop, sK(j + 1), lane);
      fwd_softmax<MASKED>(s, m, l, alpha, p, a.scale_log2, km);
      if constexpr (decltype(has_next)::value) {
        s[0] = sn[0];
        s[1] = sn[1];
      }
    }
    // The softmax results are complete here: without this the compiler may
    // sink the softmax below the barrier.
    asm volatile("" ::"v"(p[0][0]), "v"(p[0][1]), "v"(p[1][0]), "v"(p[1][1]), "v"(alpha), "v"(l));
    wait_vmem();
    __syncthreads();
  };
  using F = std::false_type;
  using Tr = std::true_type;
  // Full tiles come first in the list, then partial ones.  The first and the
  // last step are peeled, and the steps between run in two loops (full,
  // partial) rather than one loop with a branch, which would make the
  // compiler copy every accumulator at the merge.
  if (n > 0) {
    if (n > 1) {
      if (nfull > 0) step(0, F{}, F{}, Tr{});
      else step(0, Tr{}, F{}, Tr{});
      int j = 1;
      for (; j < min(nfull, n - 1); ++j) step(j, F{}, Tr{}, Tr{});
      for (; j < n - 1; ++j) step(j, Tr{}, Tr{}, Tr{});
      if (n - 1 < nfull) step(n - 1, F{}, Tr{}, F{});
      else step(n - 1, Tr{}, Tr{}, F{});
    } else {
      if (nfull > 0) step(0, F{}, F{}, F{});
      else step(0, Tr{}, F{}, F{});
    }
    fwd_pv<D>(o, p, alpha, sV(n - 1), lane);
    __syncthreads();  // every wave is done with V(n-1) before O goes to LDS
  }

  // Epilogue: normalise; O (bf16) goes through LDS so that its rows leave
  // as whole contiguous segments; LSE in natural log.
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

template <int D, bool ROPE>
hipError_t launch_fwd_d(const FwdArgs& a, int wgh, unsigned nblk, hipStream_t stream) {
  switch (wgh) {
    case 4:
      hipLaunchKernelGGL((fwd_kernel<D, 4, ROPE>), dim3(nblk), dim3(256), 0, stream, a);
      break;
    case 2:
      hipLaunchKernelGGL((fwd_kernel<D, 2, ROPE>), dim3(nblk), dim3(256), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((fwd_kernel<D, 1, ROPE>), dim3(nblk), dim3(256), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int fwd_wg_heads(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1); }

hipError_t launch_fwd(const FwdArgs& a, int D, int B, hipStream_t stream) {
  const int wgh = fwd_wg_heads(a.G);
  const unsigned nblk = (unsigned)((int64_t)B * a.map.nqt * (a.Hq / wgh));
  if (a.rope_log2_base != 0.f)
    return D == 128 ? launch_fwd_d<128, true>(a, wgh, nblk, stream) : launch_fwd_d<64, true>(a, wgh, nblk, stream);
  return D == 128 ? launch_fwd_d<128, false>(a, wgh, nblk, stream) : launch_fwd_d<64, false>(a, wgh, nblk, stream);
}

}  // namespace pba
