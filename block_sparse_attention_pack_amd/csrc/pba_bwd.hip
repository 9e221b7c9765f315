// Backward kernels of packed branch-aware attention (no atomics).
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
//             wave = 32 queries of one head.  It forms Delta from dO and O in
//             registers and writes Delta and the log2-domain LSE (0 where the
//             row sees nothing) for bwd_dkdv, then walks the query tile's key
//             tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//   bwd_dkdv  key-major, on a map with 64-query x 128-key tiles.  A
//             workgroup = one key tile x one kv group, one wave = 32 keys whose
//             K and V stay in registers.  It walks the key tile's query tiles
//             and, for each q head of the group, S = Q K^T, dP = dO V^T,
//             dV^T += dO^T P, dK^T += Q^T dS, summing over the group's heads.
//
// dQ and dK / dV are each owned by exactly one workgroup, so they are written
// once, in bf16, with no accumulator pass (fp32 atomics into a dQ buffer are
// capped by the L2 atomic rate far below the MFMA rate at these shapes).
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

// One key tile for one wave of bwd_dq (64 keys x 32 queries).  Key
// j = k0 + 32*aa + 8*(r/4) + 4*hi + r%4 sits in register r of s[aa]; the
// mask parameters are those of the forward (see fwd_tile).
template <int D, bool MASK>
__device__ __forceinline__ void dq_tile(f32x16 (&dq)[D / 32], const bf16x8 (&qop)[D / 16],
                                        const bf16x8 (&dop)[D / 16], float l2, float delta,
                                        const bf16* __restrict__ sk, const bf16* __restrict__ sv, float scale_log2,
                                        int lim, int lo, int pc, int plen, int lane) {
  using C = BwdCfg<D>;
  const int l32 = lane & 31, hi = lane >> 5;
  // The two 32-key halves one after the other (fewer live registers).
#pragma unroll
  for (int aa = 0; aa < 2; ++aa) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < C::NS; ++st) {
      const bf16x8 kop = *(const bf16x8*)(sk + prow(32 * aa + l32) * C::STR + 16 * st + 8 * hi);
      s = mfma32(kop, qop[st], s);
      const bf16x8 vop = *(const bf16x8*)(sv + prow(32 * aa + l32) * C::STR + 16 * st + 8 * hi);
      dp = mfma32(vop, dop[st], dp);
    }
    sched_fence();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -l2));
      if (MASK) {
        const int off = 32 * aa + 8 * (r >> 2) + (r & 3);
        const bool ok = off <= lim && (off >= lo || (unsigned)(off + pc) < (unsigned)plen);
        p = ok ? p : 0.f;
      }
      s[r] = p * (dp[r] - delta);
    }
    const bf16x8 ds[2] = {pack8(s, 0), pack8(s, 8)};
    sched_fence();
    // dQ^T += K^T dS^T: A = K^T by transpose reads, B = dS^T (key order of
    // the accumulator layout).
#pragma unroll
    for (int e = 0; e < C::NE; ++e) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = 32 * aa + 16 * u + 4 * hi;
        const bf16x8 kt = lds_tr8p(sk, C::STR, r0, r0 + 8, 32 * e, lane);
        dq[e] = mfma32(kt, ds[u], dq[e]);
      }
    }
  }
}

template <int D, int WGH>
__global__ void __launch_bounds__(256, 2) bwd_dq(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) bf16 sK[2][64 * C::STR];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][64 * C::STR];

  const MapView& mp = a.qmap;
  if (cptr(mp.status)[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int nhg = a.Hq / WGH;
  const int item = cptr(mp.q_order)[blockIdx.x / nhg];
  const int b = item / mp.nqt, qt = item % mp.nqt;
  const int h = (blockIdx.x % nhg) * WGH + (w % WGH);
  const int g = h / a.G;
  const int S = a.S, Hq = a.Hq, Hkv = a.Hkv;
  const int qi = qt * (32 * (4 / WGH)) + (w / WGH) * 32 + l32;
  const int qc = min(qi, S - 1);

  // Q^T and dO^T as B operands; Delta = rowsum(dO * O) from the same lanes.
  bf16x8 qop[C::NS], dop[C::NS];
  float delta = 0.f;
  {
    const int64_t off = (((int64_t)b * S + qc) * Hq + h) * D + 8 * hi;
#pragma unroll
    for (int st = 0; st < C::NS; ++st) {
      qop[st] = *(const bf16x8*)(a.q + off + 16 * st);
      dop[st] = *(const bf16x8*)(a.dout + off + 16 * st);
      const bf16x8 ov = *(const bf16x8*)(a.o + off + 16 * st);
#pragma unroll
      for (int t = 0; t < 8; ++t) delta += (float)dop[st][t] * (float)ov[t];
    }
    delta += wave_half_swap(delta);
  }
  const int4 wv = reinterpret_cast<const int4*>(mp.tok_win)[(int64_t)b * S + qc];
  const int wlo = qi < S ? wv.x : qi + 1, wplo = qi < S ? wv.y : 0, wphi = qi < S ? wv.z : 0;
  const float lse = a.lse[((int64_t)b * Hq + h) * S + qc];
  // log2-domain LSE; a row that sees no key (LSE = -inf) is masked on every
  // tile it meets, and 0 keeps its arithmetic finite.
  const float l2 = lse == kNegInf ? 0.f : lse * kLog2e;

  const int64_t lrow = (int64_t)b * mp.nqt + qt;
  const cint_ptr cnt = cptr(mp.q2k_cnt) + lrow * 2;
  const int n = min(max(cnt[0] + cnt[1], 0), mp.nkt);
  const int nfull = min(max(cnt[0], 0), n);
  const cint_ptr list = cptr(mp.q2k_idx) + lrow * mp.nkt;

  const int kvstride = Hkv * D;
  const bf16* kb = a.k + ((int64_t)b * S * Hkv + g) * D;
  const bf16* vb = a.v + ((int64_t)b * S * Hkv + g) * D;
  // One stager per staged tensor: two DMA streams sharing offset registers
  // make the compiler wait for both before every LDS read of the tile.
  const Stager<D, C::STR> kst(tid, kvstride), vst(tid, kvstride);

  f32x16 dq[C::NE];
#pragma unroll
  for (int e = 0; e < C::NE; ++e) dq[e] = f32x16{};

  if (n > 0) {
    const int k0 = min(max(list[0], 0), mp.nkt - 1) * 64;
    kst.stage(sK[0], kb + (int64_t)k0 * kvstride, S - k0);
    vst.stage(sV[0], vb + (int64_t)k0 * kvstride, S - k0);
  }
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < n; ++j) {
    const int kt = min(max(list[j], 0), mp.nkt - 1);
    const int buf = j & 1;
    if (j + 1 < n) {
      const int k0 = min(max(list[j + 1], 0), mp.nkt - 1) * 64;
      kst.stage(sK[buf ^ 1], kb + (int64_t)k0 * kvstride, S - k0);
      vst.stage(sV[buf ^ 1], vb + (int64_t)k0 * kvstride, S - k0);
    }
    if (j < nfull) {
      dq_tile<D, false>(dq, qop, dop, l2, delta, sK[buf], sV[buf], a.scale_log2, 0, 0, 0, 0, lane);
    } else {
      const int jb = kt * 64 + 4 * hi;
      dq_tile<D, true>(dq, qop, dop, l2, delta, sK[buf], sV[buf], a.scale_log2, qi - jb, wlo - jb, jb - wplo,
                       wphi - wplo, lane);
    }
    wait_vmem();
    __syncthreads();
  }

  // (Delta and LSE2 are stored only now: a store still in flight when the
  // loop reuses its data registers would make every tile wait for memory.)
  if (qi < S && hi == 0) {
    a.delta[((int64_t)b * Hq + h) * S + qi] = delta;
    a.lse2[((int64_t)b * Hq + h) * S + qi] = l2;
  }
  if (qi < S) {
    bf16* row = a.dq + (((int64_t)b * S + qi) * Hq + h) * D + 4 * hi;
#pragma unroll
    for (int e = 0; e < C::NE; ++e) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (bf16)(dq[e][4 * rg + t] * a.scale);
        *(bf16x4*)(row + 32 * e + 8 * rg) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_dkdv
// ---------------------------------------------------------------------------

// One (query tile, q head) step for one wave of bwd_dkdv: 64 queries x the
// wave's 32 keys.  Query q = q0 + 32*c + 8*(r/4) + 4*hi + r%4 sits in
// register r of s[c]; the lane's key kj is seen by queries [kj, qend).
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_step(f32x16 (&dkt)[D / 32], f32x16 (&dvt)[D / 32], const bf16x8 (&kop)[D / 16],
                                          const bf16x8 (&vop)[D / 16], const bf16* __restrict__ sq,
                                          const bf16* __restrict__ sdo, const float* __restrict__ sl,
                                          const float* __restrict__ sd, float scale_log2, int qrel, int qlim,
                                          int lane) {
  using C = BwdCfg<D>;
  const int l32 = lane & 31, hi = lane >> 5;
  f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int st = 0; st < C::NS; ++st) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 qa = *(const bf16x8*)(sq + prow(32 * c + l32) * C::STR + 16 * st + 8 * hi);
      s[c] = mfma32(qa, kop[st], s[c]);
      const bf16x8 da = *(const bf16x8*)(sdo + prow(32 * c + l32) * C::STR + 16 * st + 8 * hi);
      dp[c] = mfma32(da, vop[st], dp[c]);
    }
  }
  sched_fence();
  bf16x8 pb[2][2], db[2][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int qr = 32 * c + 8 * rg + 4 * hi;  // rows qr .. qr+3 in registers 4*rg .. 4*rg+3
      const f32x4 lv = *(const f32x4*)(sl + qr);
      const f32x4 dv = *(const f32x4*)(sd + qr);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 4 * rg + t;
        float p = fast_exp2(__builtin_fmaf(s[c][r], scale_log2, -lv[t]));
        if (MASK) p = (unsigned)(qr + t - qrel) < (unsigned)qlim ? p : 0.f;
        s[c][r] = p;
        dp[c][r] = p * (dp[c][r] - dv[t]);
      }
    }
    pb[c][0] = pack8(s[c], 0);
    pb[c][1] = pack8(s[c], 8);
    db[c][0] = pack8(dp[c], 0);
    db[c][1] = pack8(dp[c], 8);
  }
  sched_fence();
  // dV^T += dO^T P and dK^T += Q^T dS (reduction over queries, in the
  // register order of P / dS).
#pragma unroll
  for (int e = 0; e < C::NE; ++e) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = 32 * c + 16 * u + 4 * hi;
        const bf16x8 doT = lds_tr8p(sdo, C::STR, r0, r0 + 8, 32 * e, lane);
        dvt[e] = mfma32(doT, pb[c][u], dvt[e]);
        const bf16x8 qT = lds_tr8p(sq, C::STR, r0, r0 + 8, 32 * e, lane);
        dkt[e] = mfma32(qT, db[c][u], dkt[e]);
      }
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256, 1) bwd_dkdv(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) bf16 sQ[2][64 * C::STR];
  __shared__ __attribute__((aligned(1024))) bf16 sDO[2][64 * C::STR];
  __shared__ __attribute__((aligned(16))) float sL[2][64], sD[2][64];

  const MapView& mp = a.kmap;
  if (cptr(mp.status)[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int Hkv = a.Hkv, G = a.G, S = a.S, Hq = a.Hq;
  const int item = cptr(mp.k_order)[blockIdx.x / Hkv];
  const int g = blockIdx.x % Hkv;
  const int b = item / mp.nkt, kt = item % mp.nkt;
  const int kj = kt * 128 + 32 * w + l32;  // this lane's key
  const int kc = min(kj, S - 1);

  // K and V of the lane's key as B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kop[C::NS], vop[C::NS];
  {
    const int64_t off = (((int64_t)b * S + kc) * Hkv + g) * D + 8 * hi;
#pragma unroll
    for (int st = 0; st < C::NS; ++st) {
      kop[st] = *(const bf16x8*)(a.k + off + 16 * st);
      vop[st] = *(const bf16x8*)(a.v + off + 16 * st);
    }
  }
  const int qend = kj < S ? reinterpret_cast<const int4*>(mp.tok_win)[(int64_t)b * S + kc].w : kj;

  const int64_t lrow = (int64_t)b * mp.nkt + kt;
  const cint_ptr cnt = cptr(mp.k2q_cnt) + lrow * 2;
  const int n = min(max(cnt[0] + cnt[1], 0), mp.nqt);
  const int nfull = min(max(cnt[0], 0), n);
  const cint_ptr list = cptr(mp.k2q_idx) + lrow * mp.nqt;

  // The next step's Q and dO tiles and its 64 LSE2 / Delta values are
  // loaded into registers while the current step computes, and written to
  // the other LDS buffer after the current step's last LDS read.
  const int qstride = Hq * D;
  using Reg = RegStager<D, C::STR>;
  const Reg qst(tid, qstride);
  u32x4 rq[Reg::CH], rdo[Reg::CH];
  float rl = 0.f, rd = 0.f;
  auto load_step = [&](int i, int hh) {
    const int qt = min(max(list[i], 0), mp.nqt - 1), h = g * G + hh;
    const int64_t toff = ((int64_t)b * S + qt * 64) * qstride + (int64_t)h * D;
    qst.load(rq, a.q + toff, S - qt * 64);
    qst.load(rdo, a.dout + toff, S - qt * 64);
    if (tid < 64) {
      const int q = qt * 64 + tid;
      const int64_t ro = ((int64_t)b * Hq + h) * S + min(q, S - 1);
      rl = q < S ? a.lse2[ro] : 0.f;
      rd = q < S ? a.delta[ro] : 0.f;
    }
  };
  auto store_step = [&](int buf) {
    Reg::store(sQ[buf], rq, tid);
    Reg::store(sDO[buf], rdo, tid);
    if (tid < 64) {
      sL[buf][tid] = rl;
      sD[buf][tid] = rd;
    }
  };

  f32x16 dkt[C::NE], dvt[C::NE];
#pragma unroll
  for (int e = 0; e < C::NE; ++e) dkt[e] = dvt[e] = f32x16{};

  if (n > 0) {
    load_step(0, 0);
    store_step(0);
  }
  __syncthreads();
  int buf = 0;
  for (int i = 0; i < n; ++i) {
    const int qt = min(max(list[i], 0), mp.nqt - 1);
    const bool masked = i >= nfull;
    for (int hh = 0; hh < G; ++hh) {
      const bool next_same = hh + 1 < G, next_tile = !next_same && i + 1 < n;
      if (next_same) load_step(i, hh + 1);
      else if (next_tile) load_step(i + 1, 0);
      if (!masked) {
        dkdv_step<D, false>(dkt, dvt, kop, vop, sQ[buf], sDO[buf], sL[buf], sD[buf], a.scale_log2, 0, 0, lane);
      } else {
        dkdv_step<D, true>(dkt, dvt, kop, vop, sQ[buf], sDO[buf], sL[buf], sD[buf], a.scale_log2,
                           kj - qt * 64, qend - kj, lane);
      }
      // The other buffer was last read one step ago (before the barrier).
      if (next_same || next_tile) store_step(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T.  Lane: key kj, head dims
  // 32e + 8*(r/4) + 4*hi + r%4.
  if (kj < S) {
    const int64_t off = (((int64_t)b * S + kj) * Hkv + g) * D + 4 * hi;
#pragma unroll
    for (int e = 0; e < C::NE; ++e) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 vk, vv;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          vk[t] = (bf16)(dkt[e][4 * rg + t] * a.scale);
          vv[t] = (bf16)dvt[e][4 * rg + t];
        }
        *(bf16x4*)(a.dk + off + 32 * e + 8 * rg) = vk;
        *(bf16x4*)(a.dv + off + 32 * e + 8 * rg) = vv;
      }
    }
  }
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
    const unsigned nblk = (unsigned)((int64_t)a.B * a.kmap.nkt * a.Hkv);
    bwd_dkdv<D><<<nblk, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, int stages, hipStream_t stream) {
  return D == 128 ? launch_bwd_d<128>(a, stages, stream) : launch_bwd_d<64>(a, stages, stream);
}

}  // namespace pba
