// Backward kernels of packed branch-aware attention.
//
//   bwd_delta   Delta[b,h,i] = sum_d dO[b,i,h,d] * O[b,i,h,d] (fp32) and zero
//               the fp32 dQ accumulator (one streaming pass, HBM-bound)
//   bwd_main    per (row, 128-key tile, kv head): walks the key tile's visit
//               list of 64-query tiles and, for every q head of the group,
//               recomputes P = exp(scale q.k - LSE) (masked on partial tiles
//               only), then dV += P^T dO, dP = dO V^T, dS = P (dP - Delta),
//               dK += scale dS^T Q, and adds scale dS K into the dQ
//               accumulator with fp32 atomics
//   bwd_dq_cvt  fp32 dQ accumulator -> bf16 dQ
//
// dS = P (dP - rowsum(dO * O)) is the softmax Jacobian written with the
// forward's output (rowsum(P * dP) = rowsum(dO * O) for each query row).
//
// Layout: each of the 4 waves owns 32 keys.  Scores are computed as
// S = Q K^T with queries on MFMA rows and the wave's keys on MFMA columns, so
// P and dS in the accumulator layout are directly the B operands of
// dV^T = dO^T P and dK^T = Q^T dS; dO^T and Q^T are read with LDS transpose
// reads from the row-major tiles.  dS goes through LDS (stored [key][query])
// so that each wave can form a 32-wide slice of dQ = dS K over all 128 keys.
#include "pba_tile.h"

namespace pba {
namespace {

constexpr float kNegInf = -__builtin_inff();

template <int D>
__global__ void __launch_bounds__(256) bwd_delta(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                 float* __restrict__ delta, float* __restrict__ dq_acc,
                                                 int64_t nchunks, int S, int Hq, const int32_t* __restrict__ status) {
  if (status[0] != 0) return;
  constexpr int CPR = D / 8;  // 16-byte chunks per (token, head)
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float acc = 0.f;
  if (c < nchunks) {
    const bf16x8 x = *(const bf16x8*)(o + 8 * c);
    const bf16x8 y = *(const bf16x8*)(dout + 8 * c);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += (float)x[t] * (float)y[t];
    *(float4*)(dq_acc + 8 * c) = make_float4(0.f, 0.f, 0.f, 0.f);
    *(float4*)(dq_acc + 8 * c + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (c < nchunks && (c % CPR) == 0) {
    const int64_t row = c / CPR;  // (b, s, h)
    const int h = (int)(row % Hq);
    const int64_t bs = row / Hq;
    const int s = (int)(bs % S);
    const int64_t bb = bs / S;
    delta[(bb * Hq + h) * S + s] = acc;
  }
}

__global__ void __launch_bounds__(256) bwd_dq_cvt(const float* __restrict__ dq_acc, bf16* __restrict__ dq,
                                                  int64_t nchunks, const int32_t* __restrict__ status) {
  if (status[0] != 0) return;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const float4 x0 = *(const float4*)(dq_acc + 8 * c);
  const float4 x1 = *(const float4*)(dq_acc + 8 * c + 4);
  bf16x8 r;
  r[0] = (bf16)x0.x; r[1] = (bf16)x0.y; r[2] = (bf16)x0.z; r[3] = (bf16)x0.w;
  r[4] = (bf16)x1.x; r[5] = (bf16)x1.y; r[6] = (bf16)x1.z; r[7] = (bf16)x1.w;
  *(bf16x8*)(dq + 8 * c) = r;
}

template <int D>
__global__ void __launch_bounds__(256, 1) bwd_main(BwdArgs a) {
  constexpr int NS = D / 16;
  constexpr int NE = D / 32;
  constexpr int STR = D + 8;       // Q / dO tile row stride (elements)
  constexpr int DSTR = 64 + 8;     // dS^T tile row stride (elements)
  constexpr int CH = 64 * D / 8 / 256;  // 16-byte chunks per thread per tile
  constexpr int NQB = NE / 2;      // dQ 32x32 blocks per wave (2 query blocks x NE head blocks / 4 waves)
  __shared__ __attribute__((aligned(16))) bf16 sQ[2][64 * STR];
  __shared__ __attribute__((aligned(16))) bf16 sDO[2][64 * STR];
  __shared__ __attribute__((aligned(16))) bf16 sDS[128 * DSTR];
  __shared__ float sL[2][64], sDl[2][64];

  const MapView& mp = a.map;
  if (mp.status[0] != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int S = a.S, Hq = a.Hq, Hkv = a.Hkv, G = a.G;
  const int kvw = kt * 128 + 32 * w;  // this wave's first key
  const int kj = kvw + l32;           // this lane's key

  // K and V of the lane's key as B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kop[NS], vop[NS];
  int qend = kj;
  if (kj < S) {
    const int64_t off = (((int64_t)b * S + kj) * Hkv + g) * D + 8 * hi;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      kop[st] = *(const bf16x8*)(a.k + off + 16 * st);
      vop[st] = *(const bf16x8*)(a.v + off + 16 * st);
    }
    qend = mp.tok_win[((int64_t)b * S + kj) * 4 + 3];
  } else {
#pragma unroll
    for (int st = 0; st < NS; ++st) kop[st] = vop[st] = bf16x8{};
  }

  // K of the whole key tile as the B operand of dQ = dS K for this wave's
  // dQ blocks: staged through LDS (the Q buffers, 128 rows) and read
  // column-wise.  Block j of this wave: query block qb(j), head block eb(j).
  bf16* sKt = &sQ[0][0];
  {
    constexpr int KCH = 128 * D / 8 / 256;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), c8 = c % (D / 8);
      const int kk = kt * 128 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < S) v = *(const uint4*)(a.k + (((int64_t)b * S + kk) * Hkv + g) * D + 8 * c8);
      *(uint4*)&sKt[r * STR + 8 * c8] = v;
    }
  }
  __syncthreads();
  bf16x8 ktop[NQB][8];
  int qb[NQB], eb[NQB];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    if (NE == 4) { qb[j] = j; eb[j] = w; } else { qb[j] = w >> 1; eb[j] = w & 1; }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int r0 = 16 * st + 8 * hi;
      ktop[j][st] = lds_tr8(sKt, STR, r0, r0 + 4, 32 * eb[j], lane);
    }
  }
  __syncthreads();

  const int64_t lrow = (int64_t)b * mp.nkt + kt;
  const int nt = min(max(mp.k2q_cnt[lrow * 2] + mp.k2q_cnt[lrow * 2 + 1], 0), mp.nqt);
  const int nfull = min(max(mp.k2q_cnt[lrow * 2], 0), nt);
  const int32_t* list = mp.k2q_idx + lrow * mp.nqt;
  const int nsteps = nt * G;

  f32x16 dkt[NE], dvt[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) dkt[e] = dvt[e] = f32x16{};

  uint4 rq[CH], rdo[CH];
  float rl = 0.f, rd = 0.f;
  auto gload = [&](int step) {
    const int qt = list[step / G], h = g * G + step % G;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), c8 = c % (D / 8);
      const int qi = qt * 64 + r;
      if ((unsigned)qi < (unsigned)S) {
        const int64_t off = (((int64_t)b * S + qi) * Hq + h) * D + 8 * c8;
        rq[i] = *(const uint4*)(a.q + off);
        rdo[i] = *(const uint4*)(a.dout + off);
      } else {
        rq[i] = rdo[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 64) {
      const int qi = qt * 64 + tid;
      if ((unsigned)qi < (unsigned)S) {
        rl = a.lse[((int64_t)b * Hq + h) * S + qi] * kLog2e;
        rd = a.delta[((int64_t)b * Hq + h) * S + qi];
      } else {
        rl = 0.f;
        rd = 0.f;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + 256 * i, r = c / (D / 8), c8 = c % (D / 8);
      *(uint4*)&sQ[buf][r * STR + 8 * c8] = rq[i];
      *(uint4*)&sDO[buf][r * STR + 8 * c8] = rdo[i];
    }
    if (tid < 64) {
      sL[buf][tid] = rl;
      sDl[buf][tid] = rd;
    }
  };

  if (nsteps > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const int li = step / G;
    const int qt = list[li], h = g * G + step % G;
    const bool partial = li >= nfull;
    if (step + 1 < nsteps) gload(step + 1);

    // S = Q K^T and dP = dO V^T: rows = 64 queries (2 blocks), columns = keys.
    f32x16 sc[2], dp[2];
    sc[0] = sc[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 qa = *(const bf16x8*)&sQ[buf][(32 * c + l32) * STR + 16 * st + 8 * hi];
        sc[c] = mfma32(qa, kop[st], sc[c]);
        const bf16x8 da = *(const bf16x8*)&sDO[buf][(32 * c + l32) * STR + 16 * st + 8 * hi];
        dp[c] = mfma32(da, vop[st], dp[c]);
      }
    }

    // P and dS (queries along registers, this lane's key fixed).
    bf16x8 pb[2][2], db[2][2];  // [query block][k-step half]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 32 * c + 8 * (r >> 2) + 4 * hi + (r & 3);
        float p = fast_exp2(sc[c][r] * a.scale_log2 - sL[buf][qr]);
        if (partial) {
          const int qi = qt * 64 + qr;
          const bool ok = (unsigned)(qi - kj) < (unsigned)(qend - kj);
          p = ok ? p : 0.f;
        }
        sc[c][r] = p;
        dp[c][r] = p * (dp[c][r] - sDl[buf][qr]);
      }
      pb[c][0] = pack8(sc[c], 0);
      pb[c][1] = pack8(sc[c], 8);
      db[c][0] = pack8(dp[c], 0);
      db[c][1] = pack8(dp[c], 8);
    }

    // dV^T += dO^T P and dK^T += Q^T dS (k = queries, in P's register order).
#pragma unroll
    for (int e = 0; e < NE; ++e) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 32 * c + 16 * u + 4 * hi;
          const bf16x8 doT = lds_tr8(sDO[buf], STR, r0, r0 + 8, 32 * e, lane);
          dvt[e] = mfma32(doT, pb[c][u], dvt[e]);
          const bf16x8 qT = lds_tr8(sQ[buf], STR, r0, r0 + 8, 32 * e, lane);
          dkt[e] = mfma32(qT, db[c][u], dkt[e]);
        }
      }
    }

    // dS^T -> LDS: this wave's 32 key rows, 4 consecutive queries per write.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = db[c][rg >> 1][4 * (rg & 1) + t];
        *(bf16x4*)&sDS[(32 * w + l32) * DSTR + 32 * c + 8 * rg + 4 * hi] = v;
      }
    }
    __syncthreads();

    // dQ slice = scale * dS K over the tile's 128 keys, added atomically.
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int r0 = 16 * st + 8 * hi;
        const bf16x8 dsa = lds_tr8(sDS, DSTR, r0, r0 + 4, 32 * qb[j], lane);
        acc = mfma32(dsa, ktop[j][st], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qt * 64 + 32 * qb[j] + 8 * (r >> 2) + 4 * hi + (r & 3);
        if ((unsigned)qi < (unsigned)S)
          atomicAdd(a.dq_acc + (((int64_t)b * S + qi) * Hq + h) * D + 32 * eb[j] + l32, acc[r] * a.scale);
      }
    }

    if (step + 1 < nsteps) sstore(buf ^ 1);
    __syncthreads();
  }

  // dK = scale * dK^T^T, dV = dV^T^T (bf16).  Lane: key kj, head dims
  // 32e + 8*(r/4) + 4*hi + r%4.
  if (kj < S) {
    const int64_t off = (((int64_t)b * S + kj) * Hkv + g) * D + 4 * hi;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
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
hipError_t launch_bwd_stage_d(const BwdArgs& a, int stage, hipStream_t stream) {
  const int64_t nchunks = (int64_t)a.B * a.S * a.Hq * D / 8;
  const unsigned nb = (unsigned)((nchunks + 255) / 256);
  if (stage & kBwdPre)
    bwd_delta<D><<<nb, 256, 0, stream>>>(a.o, a.dout, a.delta, a.dq_acc, nchunks, a.S, a.Hq, a.map.status);
  if (stage & kBwdMain) bwd_main<D><<<dim3(a.map.nkt, a.Hkv, a.B), 256, 0, stream>>>(a);
  if (stage & kBwdFin) bwd_dq_cvt<<<nb, 256, 0, stream>>>(a.dq_acc, a.dq, nchunks, a.map.status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, int stages, hipStream_t stream) {
  return D == 128 ? launch_bwd_stage_d<128>(a, stages, stream) : launch_bwd_stage_d<64>(a, stages, stream);
}

}  // namespace pba
