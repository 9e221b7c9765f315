// Backward kernels of packed branch-aware attention (no atomic accumulation).
//
// For the loss <dO, O> with P = softmax(scale * Q K^T under the mask):
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - Delta),  dQ = scale dS K,
//   dK = scale dS^T Q,  where Delta_i = rowsum(dO * O)_i = rowsum(P * dP)_i
// (the softmax Jacobian written with the forward's output).  P is recomputed
// from the forward's log-sum-exp.  Only the tiles the block map marks full
// or partial are visited; the mask is applied on partial tiles only.
//
//   bwd_dq    query-major, on the map of the forward's tile shape.  A
//             workgroup = one query tile x WGH q heads of one kv group, one
//             wave = 32 queries of one head.  Its prologue stages the Q and
//             dO blocks (O straight into registers), forms
//             Delta = rowsum(dO * O) and stages the first K/V tile; it writes
//             -Delta and -LSE / scale (0 where the row sees nothing) for
//             bwd_dkdv.  Then it walks the query tile's key tiles:
//             S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T, the two
//             32-key halves of a tile staggered.
//   bwd_dkdv  key-major, on a map with 64-query x 128-key tiles.  A
//             workgroup = one key tile x one kv group, 8 waves (32 keys x one
//             32-query half each); K and V of the 128 keys stay in LDS, a
//             wave's K operands, dK^T and dV^T in registers.  It walks the
//             key tile's query tiles and, for each q head of the group,
//             S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS, summing
//             over the group's heads; the two query halves' partial sums meet
//             in LDS at the end.
//             Key tiles with a list longer than the average load of one
//             workgroup slot (the prompt tiles of a pack shared by many
//             responses) are split between two workgroups, whose fp32 sums
//             meet in the workspace: the second to finish adds them.
//
// dQ and dK / dV are each owned by exactly one workgroup, so they are written
// once, in bf16, with no accumulator pass (fp32 atomics into a dQ buffer are
// capped by the L2 atomic rate far below the MFMA rate at these shapes).
#include <type_traits>

#include "pba_tile.h"

namespace pba {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int D>
struct BwdCfg {
  static constexpr int NS = D / 16;    // MFMA k-steps over the head dim
  static constexpr int NE = D / 32;    // 32-wide blocks of the head dim
  static constexpr int STR = D + 8;    // staged tile row stride (elements)
};

// ---------------------------------------------------------------------------
// bwd_dq
// ---------------------------------------------------------------------------

// One key tile for one wave of bwd_dq (64 keys x 32 queries), hand-
// scheduled.  Per 32-key half aa: S^T = K Q^T and dP^T = V dO^T (16 MFMAs),
// dS^T = P^T (dP^T - Delta) with P^T = exp2(S^T * scale_log2 - LSE2)
// (vector ALU), then dQ^T += K^T dS^T (8 MFMAs, K^T by transpose reads).
// The halves are staggered so that the vector work of one half runs
// between the MFMAs of the other: S/dP of half 0, S/dP of half 1 with the
// dS of half 0, dQ of half 0 with the dS of half 1, dQ of half 1.  Every
// MFMA's LDS operand is read two MFMAs ahead.  Key
// j = k0 + 32*aa + 8*(r/4) + 4*hi + r%4 sits in register r of s[aa]; the
// mask parameters are those of the forward.
template <int D, bool MASK>
__device__ __forceinline__ void dq_tile(f32x16 (&dq)[D / 32], const bf16x8 (&qop)[D / 16],
                                        const bf16x8 (&dop)[D / 16], float l2, float delta,
                                        const bf16* __restrict__ sk, const bf16* __restrict__ sv, float scale_log2,
                                        KeyMask km, int lane) {
  using C = BwdCfg<D>;
  constexpr int NSD = 2 * C::NS;    // S and dP MFMAs of one half
  constexpr int NDQ = 2 * C::NE;    // dQ MFMAs of one half
  constexpr int N = 2 * NSD + 2 * NDQ;
  const int l32 = lane & 31, hi = lane >> 5;
  auto operand = [&](int i) __attribute__((always_inline)) -> bf16x8 {
    if (i < 2 * NSD) {  // S (even) / dP (odd) of half i / NSD, k-step (i % NSD) / 2
      const int aa = i / NSD, st = (i % NSD) >> 1;
      const bf16* t = (i & 1) ? sv : sk;
      return *(const bf16x8*)(t + prow(32 * aa + l32) * C::STR + 16 * st + 8 * hi);
    }
    const int k = i - 2 * NSD, aa = k / NDQ, e = (k % NDQ) >> 1, u = k & 1;
    const int r0 = 32 * aa + 16 * u + 4 * hi;
    return lds_tr8p(sk, C::STR, r0, r0 + 8, 32 * e, lane);
  };
  // dS of score x (0..15) of half aa, in place in s[aa].
  auto dscore = [&](f32x16 (&sa)[2], f32x16 (&pa)[2], int aa, int r) __attribute__((always_inline)) {
    float p = fast_exp2(__builtin_fmaf(sa[aa][r], scale_log2, -l2));
    if (MASK) p = keep_or_zero(mask_bit(aa ? km.hi : km.lo, 8 * (r >> 2) + (r & 3)), p);
    sa[aa][r] = p * (pa[aa][r] - delta);
  };
  f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
  bf16x8 ds[2][2];
  bf16x8 ops[3];
  ops[0] = operand(0);
  ops[1] = operand(1);
  sched_fence();
  static_for<0, N>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + 2 < N) ops[(i + 2) % 3] = operand(i + 2);
    if constexpr (i < 2 * NSD) {
      constexpr int aa = i / NSD, st = (i % NSD) >> 1;
      if constexpr (i & 1) dp[aa] = mfma32(ops[i % 3], dop[st], dp[aa]);
      else s[aa] = mfma32(ops[i % 3], qop[st], s[aa]);
      if constexpr (aa == 1) {  // dS of half 0, 16 scores over NSD slices
        constexpr int c = i - NSD;
#pragma unroll
        for (int x = 16 * c / NSD; x < 16 * (c + 1) / NSD; ++x) dscore(s, dp, 0, x);
        if constexpr (c == NSD - 1) {
          ds[0][0] = pack8(s[0], 0);
          ds[0][1] = pack8(s[0], 8);
        }
      }
    } else {
      constexpr int k = i - 2 * NSD, aa = k / NDQ, e = (k % NDQ) >> 1, u = k & 1;
      dq[e] = mfma32(ops[i % 3], ds[aa][u], dq[e]);
      if constexpr (aa == 0) {  // dS of half 1, 16 scores over NDQ slices
#pragma unroll
        for (int x = 16 * k / NDQ; x < 16 * (k + 1) / NDQ; ++x) dscore(s, dp, 1, x);
        if constexpr (k == NDQ - 1) {
          ds[1][0] = pack8(s[1], 0);
          ds[1][1] = pack8(s[1], 8);
        }
      }
    }
    sched_fence();
  });
}

// dq_tile for one 32-key half aa of a partial tile whose other half no
// query of the wave sees (its dS, hence its dQ term, is exactly zero): S^T
// and dP^T of the half, its dS^T (kmw: the half's word of the key mask),
// then its dQ^T MFMAs.
template <int D, bool MASK>
__device__ __forceinline__ void dq_half(f32x16 (&dq)[D / 32], const bf16x8 (&qop)[D / 16],
                                        const bf16x8 (&dop)[D / 16], float l2, float delta,
                                        const bf16* __restrict__ sk, const bf16* __restrict__ sv, float scale_log2,
                                        unsigned kmw, int aa, int lane) {
  using C = BwdCfg<D>;
  constexpr int NSD = 2 * C::NS;  // S and dP MFMAs
  constexpr int NDQ = 2 * C::NE;  // dQ MFMAs
  constexpr int N = NSD + NDQ;
  const int l32 = lane & 31, hi = lane >> 5;
  // prow keeps 32-row blocks in place, so the half's rows start 32*aa rows in.
  const bf16* skh = sk + 32 * aa * C::STR;
  const bf16* svh = sv + 32 * aa * C::STR;
  auto operand = [&](int i) __attribute__((always_inline)) -> bf16x8 {
    if (i < NSD) {  // S (even) / dP (odd), k-step i / 2
      const int st = i >> 1;
      return *(const bf16x8*)(((i & 1) ? svh : skh) + prow(l32) * C::STR + 16 * st + 8 * hi);
    }
    const int k = i - NSD, e = k >> 1, u = k & 1;
    const int r0 = 16 * u + 4 * hi;
    return lds_tr8p(skh, C::STR, r0, r0 + 8, 32 * e, lane);
  };
  f32x16 s = f32x16{}, dp = f32x16{};
  bf16x8 ds[2];
  bf16x8 ops[3];
  ops[0] = operand(0);
  ops[1] = operand(1);
  sched_fence();
  static_for<0, N>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + 2 < N) ops[(i + 2) % 3] = operand(i + 2);
    if constexpr (i < NSD) {
      constexpr int st = i >> 1;
      if constexpr (i & 1) dp = mfma32(ops[i % 3], dop[st], dp);
      else s = mfma32(ops[i % 3], qop[st], s);
      if constexpr (i == NSD - 1) {
        sched_fence();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -l2));
          if (MASK) p = keep_or_zero(mask_bit(kmw, 8 * (r >> 2) + (r & 3)), p);
          s[r] = p * (dp[r] - delta);
        }
        ds[0] = pack8(s, 0);
        ds[1] = pack8(s, 8);
      }
    } else {
      constexpr int k = i - NSD, e = k >> 1, u = k & 1;
      dq[e] = mfma32(ops[i % 3], ds[u], dq[e]);
    }
    sched_fence();
  });
}

template <int D, int WGH>
__global__ void __launch_bounds__(256, 2) bwd_dq(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int T = 64 * C::STR;  // elements of one K or V tile
  // K/V double buffers K(0) V(0) K(1) V(1).  The Q, dO and O blocks come
  // in through the pairs and the dQ block leaves through LDS.
  __shared__ __attribute__((aligned(1024))) bf16 lds[4 * T];
  constexpr int R = 32 * (4 / WGH);  // query rows of the workgroup
  using Blk = RowBlock<R, WGH * D * 2>;
  static_assert(Blk::BYTES <= 2 * T * 2, "a Q / dO / O block fits one buffer pair");
  auto sK = [&](int buf) { return lds + (2 * buf) * T; };
  auto sV = [&](int buf) { return lds + (2 * buf + 1) * T; };

  const MapView& mp = a.qmap;
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
  // Workgroup 0 prepares bwd_dkdv's split key tiles: the arrival counters
  // start at zero, and the number of leading work-order positions whose
  // list is more than 1.05 times the average load of a workgroup slot (all
  // visited tiles of the key-major map over the slots of one kv group) is
  // stored after them: a tile within about one workgroup prologue of the
  // average gains less from splitting than the second workgroup's prologue
  // and the exchange cost.  The work order is longest first, so those
  // positions are a prefix of it.
  if (blockIdx.x == 0) {
    for (int i = tid; i < a.nsplit * a.Hkv; i += 256) a.arrive[i] = 0;
    bool split = false;
    if (tid < a.nsplit) {
      const MapView& km = a.kmap;
      const int it = min(max(km.k_order[tid], 0), km.B * km.nkt - 1);
      const int n = min(max(km.k2q_cnt[2 * it] + km.k2q_cnt[2 * it + 1], 0), km.nqt);
      split = 20 * (int64_t)n * a.slots > 21 * (km.totals[0] + km.totals[1]);
    }
    const int nsp = __syncthreads_count(split);
    if (tid == 0) a.arrive[a.nsplit * a.Hkv] = nsp;
  }
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int nhg = a.Hq / WGH;
  const int item = min(max(order_entry, 0), mp.B * mp.nqt - 1);
  const int b = item / mp.nqt, qt = item % mp.nqt;
  const int h0 = (blockIdx.x % nhg) * WGH;
  const int hw = w % WGH, qb = w / WGH;  // this wave's head and 32-query block
  const int h = h0 + hw;
  const int g = h / a.G;
  const int S = a.S, Hq = a.Hq, Hkv = a.Hkv;
  const int q0 = qt * R;
  const int qi = q0 + qb * 32 + l32;
  const int qc = min(qi, S - 1);

  const int64_t lrow = (int64_t)b * mp.nqt + qt;
  const cint_ptr cnt = cptr(mp.q2k_cnt) + lrow * 2;
  const int n = min(max(cnt[0] + cnt[1], 0), mp.nkt);
  const int nfull = min(max(cnt[0], 0), n);
  const cint_ptr list = cptr(mp.q2k_idx) + lrow * mp.nkt;

  const int kvstride = Hkv * D;
  const bf16* kb = a.k + ((int64_t)b * S * Hkv + g) * D;
  const bf16* vb = a.v + ((int64_t)b * S * Hkv + g) * D;
  const Stager<D, C::STR> kst(tid, kvstride);  // K and V tiles have the same shape

  // Prologue in two load passes, as the Q and dO blocks and the first K/V
  // tile do not fit in LDS at once: Q and dO into the two buffer pairs (with
  // O into registers), then the first K/V tile.
  char* const pair0 = (char*)lds;             // K(0) V(0)
  char* const pair1 = (char*)(lds + 2 * T);   // K(1) V(1)
  const int qrows = min(R, S - q0), qrow_bytes = Hq * D * 2;
  const int64_t blk = ((int64_t)b * S + q0) * Hq * D + (int64_t)h0 * D;
  const int first = list[0];  // valid memory even for an empty list
  const int4 wv = reinterpret_cast<const int4*>(mp.tok_win)[(int64_t)b * S + qc];
  const float lse = a.lse[((int64_t)b * Hq + h) * S + qc];
  // Q^T and dO^T as B operands: lane holds query qi, head dims 16*st + 8*hi + 0..7.
  bf16x8 qop[C::NS], dop[C::NS];
  float delta = 0.f;
  // A query tile that visits no key tile holds only pad rows, whose dQ and
  // row values for bwd_dkdv are all 0: its row blocks are not read at all.
  if (n > 0) {
    // First load pass: the Q and dO blocks into the two buffer pairs
    // (whole-row direct loads) and, at the same time, this lane's O chunks
    // straight into registers, in the lane layout of the dO operand (query
    // row qi, head dims 16*st + 8*hi + 0..7): O is needed only for Delta.
    // Rows past S read as zeros through the resource's range.
    Blk::template load<4>(pair1, a.q + blk, qrows, qrow_bytes, w, lane);
    Blk::template load<4>(pair0, a.dout + blk, qrows, qrow_bytes, w, lane);
    u32x4 ov[C::NS];
    {
      const int r0 = q0 + qb * 32, nrows = min(32, S - r0);
      const bf16* orow = a.o + ((int64_t)b * S + r0) * Hq * D + (int64_t)h * D;
      const int nbytes = nrows > 0 ? ((nrows - 1) * Hq * D + D) * 2 : 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)orow, (short)0, nbytes, 0x00020000);
      const int voff = (l32 * Hq * D + 8 * hi) * 2;
#pragma unroll
      for (int st = 0; st < C::NS; ++st) ov[st] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 32 * st, 0, 0);
    }
    wait_vmem();
    __syncthreads();
    const int rofs = (qb * 32 + l32) * Blk::LSTR + hw * D * 2 + 16 * hi;
#pragma unroll
    for (int st = 0; st < C::NS; ++st) {
      qop[st] = *(const bf16x8*)(pair1 + rofs + 32 * st);
      dop[st] = *(const bf16x8*)(pair0 + rofs + 32 * st);
    }
    // Delta = rowsum(dO * O) from the same lanes.
#pragma unroll
    for (int st = 0; st < C::NS; ++st) {
      const bf16x8 o8 = __builtin_bit_cast(bf16x8, ov[st]);
#pragma unroll
      for (int t = 0; t < 8; ++t) delta += (float)dop[st][t] * (float)o8[t];
    }
    delta += wave_half_swap(delta);
    __syncthreads();
    // Second load pass: the first K/V tile (shared with other query tiles,
    // so mostly a cache hit).
    const int k0 = min(max(first, 0), mp.nkt - 1) * 64;
    kst.stage(sK(0), kb + (int64_t)k0 * kvstride, S - k0);
    kst.stage(sV(0), vb + (int64_t)k0 * kvstride, S - k0);
    wait_vmem();
    __syncthreads();
  }
  const int wlo = qi < S ? wv.x : qi + 1, wplo = qi < S ? wv.y : 0, wphi = qi < S ? wv.z : 0;
  // log2-domain LSE; a row that sees no key (LSE = -inf) is masked on every
  // tile it meets, and 0 keeps its arithmetic finite.
  const float l2 = lse == kNegInf ? 0.f : lse * kLog2e;

  f32x16 dq[C::NE];
#pragma unroll
  for (int e = 0; e < C::NE; ++e) dq[e] = f32x16{};
  // One visit: the next tile's loads go into the other buffer, then this
  // tile's math.  Full tiles precede partial ones in the list; a loop for
  // each keeps the dQ accumulators in place (two paths merging inside one
  // loop body would copy every accumulator per tile).
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
      const KeyMask km = key_mask(qi - jb, wlo - jb, jb - wplo, wphi - wplo);
      // Which 32-key halves some query of the wave sees (the bits of a
      // lane's 16 scores in each mask word are 0x0F0F0F0F).  A half no
      // query sees adds exactly zero, so only the other is computed (with
      // 4 q heads per workgroup, 5% of the MFMA work at Qwen3-8B-shaped
      // packs: the diagonal tiles whose second half lies after every query
      // of the block).  When neither half is seen (possible with fewer heads
      // per workgroup, whose waves cover different queries), the one-half
      // body runs with an all-zero mask and adds zero.
      const bool see0 = __builtin_amdgcn_ballot_w64((km.lo & 0x0F0F0F0Fu) != 0) != 0;
      const bool see1 = __builtin_amdgcn_ballot_w64((km.hi & 0x0F0F0F0Fu) != 0) != 0;
      if (see0 && see1)
        dq_tile<D, true>(dq, qop, dop, l2, delta, sK(buf), sV(buf), a.scale_log2, km, lane);
      else
        dq_half<D, true>(dq, qop, dop, l2, delta, sK(buf), sV(buf), a.scale_log2, see0 ? km.lo : km.hi, see0 ? 0 : 1,
                         lane);
    } else {
      dq_tile<D, false>(dq, qop, dop, l2, delta, sK(buf), sV(buf), a.scale_log2, KeyMask{0u, 0u}, lane);
    }
    wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j < nfull; ++j) visit(j, std::false_type{});
  for (; j < n; ++j) visit(j, std::true_type{});

  // For bwd_dkdv, the starting values of its dP and score accumulators
  // (stored only now: a store still in flight when the loop reuses its data
  // registers would make every tile wait for memory).
  if (qi < S && hi == 0) {
    a.dp0[((int64_t)b * Hq + h) * S + qi] = -delta;
    a.s0[((int64_t)b * Hq + h) * S + qi] = -l2 / a.scale_log2;
  }
  // With rotary inputs, dQ is rotated back to the unrotated Q's frame at
  // the query's packed position (its row is 0 where the query is pad).
  if (a.rope_log2_base != 0.f) rope_rotate_t<C::NE>(dq, (wphi - wplo) + (qi - wlo), hi, a.rope_log2_base, -1.f);
  // dQ (bf16, times the softmax scale) through LDS, free after the last
  // barrier, so that its rows leave as whole contiguous segments.
  {
    char* row = (char*)lds + (qb * 32 + l32) * Blk::LSTR + hw * D * 2 + 8 * hi;
#pragma unroll
    for (int e = 0; e < C::NE; ++e) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (bf16)(dq[e][4 * rg + t] * a.scale);
        *(bf16x4*)(row + 2 * (32 * e + 8 * rg)) = v;
      }
    }
  }
  __syncthreads();
  Blk::template store<256>(a.dq + ((int64_t)b * S + q0) * Hq * D + (int64_t)h0 * D, (const char*)lds, min(R, S - q0),
                           Hq * D * 2, tid);
}

// ---------------------------------------------------------------------------
// bwd_dkdv
// ---------------------------------------------------------------------------

// One (query tile, q head) step for one wave of bwd_dkdv: one 32-query half
// of the 64-query tile (rows q0 .. q0+31 of the staged tiles) x the wave's
// 32 keys (K operands in registers, rows k0 .. k0+31 of the resident V
// tile).  Query q0 + 8*(r/4) + 4*hi + r%4 sits in register r of s.  The
// score and dP accumulators start from -LSE / scale and -Delta (staged
// per row in s0 and dp0), so they finish as S - LSE / scale, whose
// exp2(scale_log2 * x) is P, and dP - Delta: no per-score subtraction.  On
// partial tiles (MASK) the lane's key kj is seen by queries [kj, qend): row
// index x of the tile is visible iff (unsigned)(x - qrel) < (unsigned)qlim
// (qrel = kj - the tile's first query, qlim = qend - kj).  These compares depend on the tile
// only, so the compiler keeps them in scalar lane masks across the q heads.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_step(f32x16 (&dkt)[D / 32], f32x16 (&dvt)[D / 32], const bf16x8 (&kop)[D / 16],
                                          const bf16* __restrict__ sv, int k0, const bf16* __restrict__ sq,
                                          const bf16* __restrict__ sdo, const float* __restrict__ s0,
                                          const float* __restrict__ dp0, int q0, float scale_log2, int qrel,
                                          int qlim, int lane) {
  using C = BwdCfg<D>;
  // Hand-scheduled: the S / dP MFMAs (A = Q / dO rows from LDS, B = the K
  // operands in registers / V rows from LDS), the vector work of query rows
  // 0-15 of the 32 (registers 0-7), then the dV / dK MFMAs of those rows
  // with the vector work of rows 16-31 between them, then the dV / dK MFMAs
  // of rows 16-31.  Operand reads run two MFMAs ahead.
  constexpr int NSD = 2 * C::NS, NG = 2 * C::NE, N = NSD + 2 * NG;
  const int l32 = lane & 31, hi = lane >> 5;
  struct Ops {
    bf16x8 a, b;
  };
  auto operand = [&](int i) __attribute__((always_inline)) -> Ops {
    if (i < NSD) {  // S (even) / dP (odd), k-step i / 2
      const int st = i >> 1;
      const int qo = prow(q0 + l32) * C::STR + 16 * st + 8 * hi;
      const int ko = prow(k0 + l32) * C::STR + 16 * st + 8 * hi;
      return (i & 1) ? Ops{*(const bf16x8*)(sdo + qo), *(const bf16x8*)(sv + ko)}
                     : Ops{*(const bf16x8*)(sq + qo), kop[st]};
    }
    const int k = i - NSD, u = k / NG, e = (k % NG) >> 1;  // dV (even) / dK (odd) of row half u
    const int r0 = q0 + 16 * u + 4 * hi;
    return Ops{lds_tr8p((k & 1) ? sq : sdo, C::STR, r0, r0 + 8, 32 * e, lane), bf16x8{}};
  };
  f32x16 s, dp;
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    const int qr = q0 + 8 * rg + 4 * hi;
    const f32x4 l = *(const f32x4*)(s0 + qr);
    const f32x4 d = *(const f32x4*)(dp0 + qr);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      s[4 * rg + t] = l[t];
      dp[4 * rg + t] = d[t];
    }
  }
  bf16x8 pb[2], db[2];
  // Score r (register r: query row q0 + 8*(r/4) + 4*hi + r%4).
  auto score = [&](int r) __attribute__((always_inline)) {
    const int rg = r >> 2, t = r & 3;
    float p = fast_exp2(s[r] * scale_log2);
    if (MASK) p = (unsigned)(q0 + 8 * rg + 4 * hi + t - qrel) < (unsigned)qlim ? p : 0.f;
    s[r] = p;
    dp[r] = p * dp[r];
  };
  Ops ops[3];
  ops[0] = operand(0);
  ops[1] = operand(1);
  sched_fence();
  static_for<0, N>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i + 2 < N) ops[(i + 2) % 3] = operand(i + 2);
    if constexpr (i < NSD) {
      if constexpr (i & 1) dp = mfma32(ops[i % 3].a, ops[i % 3].b, dp);
      else s = mfma32(ops[i % 3].a, ops[i % 3].b, s);
      if constexpr (i == NSD - 1) {
        sched_fence();
#pragma unroll
        for (int r = 0; r < 8; ++r) score(r);
        pb[0] = pack8(s, 0);
        db[0] = pack8(dp, 0);
      }
    } else {
      constexpr int k = i - NSD, u = k / NG, e = (k % NG) >> 1;
      if constexpr (k & 1) dkt[e] = mfma32(ops[i % 3].a, db[u], dkt[e]);
      else dvt[e] = mfma32(ops[i % 3].a, pb[u], dvt[e]);
      if constexpr (u == 0) {  // rows 16-31 (registers 8-15) spread over these NG MFMAs
#pragma unroll
        for (int r = 8 + 8 * k / NG; r < 8 + 8 * (k + 1) / NG; ++r) score(r);
        if constexpr (k == NG - 1) {
          pb[1] = pack8(s, 8);
          db[1] = pack8(dp, 8);
        }
      }
    }
    sched_fence();
  });
}

// End of bwd_dkdv: the wave of query half 1 puts its partial sums in its
// lane-private LDS slot and the partner wave (half 0) adds them to its own
// (lane: key kj, head dims 32e + 8*(r/4) + 4*hi + r%4).
template <int D>
__device__ __forceinline__ void pair_add(f32x16 (&acc)[D / 32], float* slot, int qh) {
  constexpr int NE = D / 32;
  if (qh == 1) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *(f32x4*)(slot + 16 * e + 4 * rg) =
            f32x4{acc[e][4 * rg], acc[e][4 * rg + 1], acc[e][4 * rg + 2], acc[e][4 * rg + 3]};
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 o = *(const f32x4*)(slot + 16 * e + 4 * rg);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[e][4 * rg + t] += o[t];
      }
  }
  __syncthreads();
}

// The summed block (waves of query half 0) as scale * sum in bf16 into the
// row block `rows` (LDS, row = the lane's key within the workgroup, LSTR
// bytes apart), from which the workgroup stores whole rows; with rotary
// inputs dK is first rotated back at the key's packed position.
template <int D, int LSTR>
__device__ __forceinline__ void rows_out(f32x16 (&sum)[D / 32], int qh, char* rows, int krow, int hi, float scale,
                                         bool rope, int pos, float log2_base) {
  constexpr int NE = D / 32;
  if (qh != 0) return;
  if (rope) rope_rotate_t<NE>(sum, pos, hi, log2_base, -1.f);
  char* row = rows + krow * LSTR + 8 * hi;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      bf16x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = (bf16)(sum[e][4 * rg + t] * scale);
      *(bf16x4*)(row + 2 * (32 * e + 8 * rg)) = v;
    }
  }
}

// Partial sums of one (key block, lane) in the split area: D/8 chunks of
// four floats, chunk c of lane l at (c * 64 + l) * 4 (whole 1 KB rows per
// store instruction).
template <int D>
__device__ __forceinline__ void part_store(float* p, const f32x16 (&acc)[D / 32], int lane) {
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      *(f32x4*)(p + ((4 * e + rg) * 64 + lane) * 4) =
          f32x4{acc[e][4 * rg], acc[e][4 * rg + 1], acc[e][4 * rg + 2], acc[e][4 * rg + 3]};
}

template <int D>
__device__ __forceinline__ void part_add(f32x16 (&acc)[D / 32], const float* p, int lane) {
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const f32x4 o = *(const f32x4*)(p + ((4 * e + rg) * 64 + lane) * 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[e][4 * rg + t] += o[t];
    }
}

// 8 waves, 128 keys: wave w owns the query half qh = w/4 of every 64-query
// step and the key block kb (keys 32*kb .. +31) with kb = w%4 for qh = 0 and
// kb = 3 - w%4 for qh = 1.  Waves w and w+4 share a SIMD, so a SIMD pairs
// the sub-blocks (kb, 0) and (3-kb, 1): on a tile across the causal
// diagonal the fully masked sub-blocks (keys after every query of the
// half) fall on different SIMDs than the live ones, and a wave whose
// sub-block of a partial tile is fully masked skips that step's arithmetic
// (its contribution is exactly zero), leaving its SIMD to the other wave.
// K and V of the 128 keys are staged once: each wave reads its 32 keys' K
// operands (B operands of S) into registers, while V stays in LDS (B
// operands of dP, read per step); Q, dO and the 64 rows' -LSE / scale and
// -Delta are staged by direct loads into a double buffer.  The two waves
// that share keys sum their partial dK / dV through LDS at the end.
template <int D>
__global__ void __launch_bounds__(512, 1) bwd_dkdv(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int TQ = 64 * C::STR;  // elements of one staged 64-row tile
  __shared__ __attribute__((aligned(1024))) bf16 sK[128 * C::STR];
  __shared__ __attribute__((aligned(1024))) bf16 sV[128 * C::STR];
  // Q and dO double buffers (indexed [buf] / [buf ^ 1], which lets the
  // compiler see that the tile being read and the one being loaded never
  // overlap).  After the loop they hold the exchange of partial sums: key
  // blocks 0-1 in sQ, 2-3 in sDO (2 waves x 64 lanes x D/2 fp32 each).
  __shared__ __attribute__((aligned(1024))) bf16 sQ[2][TQ];
  __shared__ __attribute__((aligned(1024))) bf16 sDO[2][TQ];
  static_assert(2 * TQ * sizeof(bf16) >= 2 * 64 * (D / 2 + 4) * sizeof(float), "exchange must fit a staging array");
  __shared__ __attribute__((aligned(16))) float sS0[2][64], sDP0[2][64];
  __shared__ int s_second;  // this workgroup is the second half of a split key tile to finish

  const MapView& mp = a.kmap;
  if (cptr(mp.status)[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int qh = w >> 2, kb = qh ? 3 - (w & 3) : (w & 3);  // query half, key block
  const int Hkv = a.Hkv, G = a.G, S = a.S, Hq = a.Hq;
  // Workgroup slots: with K split positions (counted by bwd_dq), the first
  // 2K slots take the two halves of the first K work-order positions, the
  // next ones one position each, and the nsplit - K slots at the end of the
  // grid have nothing to do.
  const int nsp = min(max(cptr(a.arrive)[a.nsplit * Hkv], 0), a.nsplit);
  const int wslot = blockIdx.x / Hkv;
  const int g = blockIdx.x % Hkv;
  if (wslot >= mp.B * mp.nkt + nsp) return;
  int pos, half = -1;
  if (wslot < 2 * nsp) {
    pos = wslot >> 1;
    half = wslot & 1;
  } else {
    pos = wslot - nsp;
  }
  const int item = min(max(cptr(mp.k_order)[pos], 0), mp.B * mp.nkt - 1);
  const int b = item / mp.nkt, kt = item % mp.nkt;
  const int kj = kt * 128 + 32 * kb + l32;  // this lane's key
  const int4 kwin = reinterpret_cast<const int4*>(mp.tok_win)[(int64_t)b * S + min(kj, S - 1)];
  const int qend = kj < S ? kwin.w : kj;

  const int64_t lrow = (int64_t)b * mp.nkt + kt;
  const cint_ptr cnt = cptr(mp.k2q_cnt) + lrow * 2;
  const int n = min(max(cnt[0] + cnt[1], 0), mp.nqt);
  const int nfull = min(max(cnt[0], 0), n);
  const cint_ptr list = cptr(mp.k2q_idx) + lrow * mp.nqt;
  // A split key tile: each half of its list goes to one workgroup.
  int i0 = 0, i1 = n;
  if (half >= 0) {
    const int n0 = (n + 1) >> 1;
    i0 = half ? n0 : 0;
    i1 = half ? n : n0;
  }

  const int kvstride = Hkv * D, qstride = Hq * D;
  const Stager<D, C::STR, 128, 8> kst(tid, kvstride);  // K and V
  const Stager<D, C::STR, 64, 8> qst(tid, qstride);    // Q and dO
  int lane4 = lane * 4;
  pin(lane4);
  if (i1 > i0) {  // (a key tile no query visits holds pad keys only: dK = dV = 0)
    const int64_t koff = ((int64_t)b * S + kt * 128) * kvstride + (int64_t)g * D;
    kst.stage(sK, a.k + koff, S - kt * 128);
    kst.stage(sV, a.v + koff, S - kt * 128);
  }
  // Staging addresses of one query tile for the group's first q head; the
  // other heads are D elements (Q, dO) or S floats (s0, dp0) further.
  // Computed once per query tile: a step only offsets the bases.
  struct TileAddr {
    const bf16* q;
    const bf16* dout;
    const float* s0;
    const float* dp0;
    int rows;  // valid rows from the tile's first on (rows past S read as zeros)
  };
  const int64_t qrow0 = (int64_t)b * S * qstride + (int64_t)(g * G) * D;
  const int64_t lrow0 = ((int64_t)b * Hq + g * G) * S;
  auto tile_addr = [&](int qt) {
    const int r0 = qt * 64;
    const int64_t o = qrow0 + (int64_t)r0 * qstride;
    return TileAddr{a.q + o, a.dout + o, a.s0 + lrow0 + r0, a.dp0 + lrow0 + r0, S - r0};
  };
  auto stage = [&](const TileAddr& t, int hh, int buf) {
    qst.stage(sQ[buf], t.q + hh * D, t.rows);
    qst.stage(sDO[buf], t.dout + hh * D, t.rows);
    if (w == 0) buffer_lds_dword(t.s0 + hh * S, t.rows, &sS0[buf][0], lane4);
    if (w == 1) buffer_lds_dword(t.dp0 + hh * S, t.rows, &sDP0[buf][0], lane4);
  };

  f32x16 dkt[C::NE], dvt[C::NE];
#pragma unroll
  for (int e = 0; e < C::NE; ++e) dkt[e] = dvt[e] = f32x16{};

  // The resident K / V tiles are read through pointers the compiler cannot
  // fold to constant addresses, so that those reads keep the alias scope of
  // dkdv_step's restrict parameters (an LDS read without one waits for
  // every outstanding global->LDS load, i.e. for the next step's tiles).
  const bf16* skp = opaque_lds(sK);
  const bf16* svp = opaque_lds(sV);
  auto tile_of = [&](int i) { return min(max(list[i], 0), mp.nqt - 1); };
  int qt_cur = tile_of(i0);  // valid memory even for an empty list
  if (i1 > i0) stage(tile_addr(qt_cur), 0, 0);
  wait_vmem();
  __syncthreads();
  int buf = 0;
  // This wave's K operands (the B operands of S = Q K^T), read once.
  bf16x8 kop[C::NS];
#pragma unroll
  for (int st = 0; st < C::NS; ++st)
    kop[st] = *(const bf16x8*)(skp + prow(32 * kb + l32) * C::STR + 16 * st + 8 * (lane >> 5));
  // Full query tiles come first in the list, then partial ones; a loop for
  // each keeps the dK / dV accumulators in place.
  auto visit = [&](int i, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int qt = qt_cur;
    // The next tile's list entry and addresses, read once per tile.
    const int qt_next = i + 1 < i1 ? tile_of(i + 1) : qt;
    const TileAddr cur = tile_addr(qt), nxt = tile_addr(qt_next);
    const int qrel = kj - qt * 64, qlim = qend - kj;
    // On a partial tile, this wave's 32 x 32 sub-block is live iff some key
    // of it is seen by some query of its half: key kj is seen by tile rows
    // [qrel, qrel + qlim).
    const bool live = !MASKED || __builtin_amdgcn_ballot_w64(qlim > 0 && qrel < 32 * qh + 32 && qrel + qlim > 32 * qh);
    for (int hh = 0; hh < G; ++hh) {
      // Prefetch the next step into the other buffer (last read one step ago).
      if (hh + 1 < G) stage(cur, hh + 1, buf ^ 1);
      else if (i + 1 < i1) stage(nxt, 0, buf ^ 1);
      if (live)
        dkdv_step<D, MASKED>(dkt, dvt, kop, svp, 32 * kb, sQ[buf], sDO[buf], sS0[buf], sDP0[buf], 32 * qh,
                             a.scale_log2, qrel, qlim, lane);
      wait_vmem();
      __syncthreads();
      buf ^= 1;
    }
    qt_cur = qt_next;
  };
  int i = i0;
  for (; i < min(nfull, i1); ++i) visit(i, std::false_type{});
  for (; i < i1; ++i) visit(i, std::true_type{});

  // Sum the two query halves: the waves of half 1 hand their partial dK^T,
  // then dV^T, to their partners through LDS (lane-private slots in the
  // Q / dO staging area); for a split key tile the two workgroups' sums then
  // meet in the workspace; the waves of half 0 write the result.  Lane: key
  // kj, head dims 32e + 8*(r/4) + 4*hi + r%4.
  float* xch = reinterpret_cast<float*>(kb < 2 ? &sQ[0][0] : &sDO[0][0]);
  const int hi = lane >> 5;
  // Slots D/2 + 4 floats apart: 16 consecutive lanes start on 16 distinct
  // 4-bank groups, so the 16-byte slot reads and writes are conflict-free.
  float* slot = xch + ((kb & 1) * 64 + lane) * (D / 2 + 4);
  // The summed dK and dV blocks (128 keys x D) go to the resident K / V
  // areas, free after the loop, and leave as whole rows.
  using Blk = RowBlock<128, D * 2>;
  static_assert(128 * Blk::LSTR <= 128 * C::STR * 2, "a dK / dV block fits the K / V area");
  const int kpos = (kwin.z - kwin.y) + (kj - kwin.x);  // the key's packed position (rows past S are not stored)
  pair_add<D>(dkt, slot, qh);
  pair_add<D>(dvt, slot, qh);
  if (half >= 0) {
    // The two workgroups of a split key tile: each leaves its fp32 sums in
    // its own half of the pair's area; the second to arrive adds the
    // other's (a + b = b + a, so the result does not depend on the order)
    // and writes dK and dV.  Each wave waits for its own stores, then one
    // agent-scope release publishes the block's stores before the counter
    // moves; the second arriver acquires before reading.
    const int64_t pair = (int64_t)pos * Hkv + g;
    float* mine = a.part + ((pair * 2 + half) * 2) * (128 * D);
    const float* other = a.part + ((pair * 2 + (half ^ 1)) * 2) * (128 * D);
    if (qh == 0) {
      part_store<D>(mine + kb * (32 * D), dkt, lane);
      part_store<D>(mine + 128 * D + kb * (32 * D), dvt, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int old = __hip_atomic_fetch_add(a.arrive + pair, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_second = old == 1;
      if (old == 1) {
        __hip_atomic_store(a.arrive + pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
    }
    __syncthreads();
    if (!s_second) return;
    if (qh == 0) {
      part_add<D>(dkt, other + kb * (32 * D), lane);
      part_add<D>(dvt, other + 128 * D + kb * (32 * D), lane);
    }
  }
  rows_out<D, Blk::LSTR>(dkt, qh, (char*)sK, 32 * kb + l32, hi, a.scale, a.rope_log2_base != 0.f, kpos,
                         a.rope_log2_base);
  rows_out<D, Blk::LSTR>(dvt, qh, (char*)sV, 32 * kb + l32, hi, 1.f, false, 0, 0.f);
  __syncthreads();
  const int krows = min(128, S - kt * 128);
  const int64_t out = ((int64_t)b * S + kt * 128) * kvstride + (int64_t)g * D;
  Blk::template store<512>(a.dk + out, (const char*)sK, krows, kvstride * 2, tid);
  Blk::template store<512>(a.dv + out, (const char*)sV, krows, kvstride * 2, tid);
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, int stages, hipStream_t stream) {
  if (stages & kBwdDq) {
    const int wgh = fwd_wg_heads(a.G);
    const unsigned nblk = (unsigned)((int64_t)a.B * a.qmap.nqt * (a.Hq / wgh));
    if (wgh == 4) bwd_dq<D, 4><<<nblk, 256, 0, stream>>>(a);
    else if (wgh == 2) bwd_dq<D, 2><<<nblk, 256, 0, stream>>>(a);
    else bwd_dq<D, 1><<<nblk, 256, 0, stream>>>(a);
  }
  if (stages & kBwdDkdv) {
    const unsigned nblk = (unsigned)(((int64_t)a.B * a.kmap.nkt + a.nsplit) * a.Hkv);
    bwd_dkdv<D><<<nblk, 512, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, int stages, hipStream_t stream) {
  return D == 128 ? launch_bwd_d<128>(a, stages, stream) : launch_bwd_d<64>(a, stages, stream);
}

}  // namespace pba
