// Block map kernels: descriptor checks, per-token ids and windows, tile
// classification, visit lists, work orders.  Integer work only; results are
// bit-exact.  Several maps of the same rows (different tile shapes) are built
// together: each stage is one launch covering all of them.
//
// The mask being summarised is the branch-aware, pack-bounded causal mask
// ("DPO Preference Packing: Dense Masks and Sparse Execution", section
// "Layout requirements"; pack boundaries as in "Pack training sequences to
// reduce padding waste", section "Preserve attention boundaries when
// examples are independent").  For a query i the visible keys are at most
// two runs, [pre_lo, pre_hi) (the prompt, seen from a later response) and
// [kv_lo, i]; a key j is seen by the queries [j, q_end).  Tiles with no
// visible pair are skipped, as a block mask skips fully masked blocks (first
// page, section "Dense and sparse execution").
//
//   map_tokens    block 0 validates the descriptors (status word, totals
//                 cleared); the other blocks locate each token's pack by
//                 binary search and write its ids and windows (reads stay in
//                 bounds even for invalid descriptors; the later stages do
//                 nothing when the status is not OK)
//   map_classify  one block per (query tile, row, map): exact count of the
//                 visible pairs of every key tile from the query windows
//   map_lists     one wave per list: ballot compaction, full then partial
//   map_order     one block per (side, map): stable sort of the tiles by
//                 visit count, descending (bitonic sort in LDS up to 2048
//                 tiles per side, a counting sort through the work area beyond)
//   map_positions (its own entry point, on a built map) aligned position
//                 ids, log-prob gather rows and the response loss mask
#include "pba_next.h"

namespace pba {
namespace {

constexpr int kThreads = 256;
constexpr int kOrderThreads = 1024;
constexpr int kOrderLds = 2048;  // tiles per side sorted in LDS; more use the chunked path

struct MapOut {
  int bm, bn, nqt, nkt;
  int32_t *tok_pack, *tok_branch, *tok_win;
  uint8_t* cls;
  int32_t *q2k_cnt, *q2k_idx, *k2q_cnt, *k2q_idx;
  int64_t* totals;
  int32_t* status;
  int32_t *q_order, *k_order, *work;
};

struct MapSet {
  int n, B, S;
  MapOut m[kMaxMapsPerBuild];
};

__device__ __forceinline__ int64_t pack_end(const pba_pack& p, const int32_t* resp_len) {
  int64_t e = (int64_t)p.start + p.prompt_len;
  for (int k = 0; k < p.n_resp; ++k) e += resp_len[p.resp_first + k];
  return e;
}

// Code of pack i's own checks (row, sign, response range, bounds); 0 if fine.
__device__ int check_pack(const pba_pack* packs, int i, const int32_t* resp_len, int n_resp_total, int B, int S) {
  const pba_pack p = packs[i];
  if (p.row < 0 || p.row >= B) return PBA_DESC_ROW;
  if (p.start < 0 || p.prompt_len < 0 || p.n_resp < 0) return PBA_DESC_NEGATIVE;
  if (p.resp_first < 0 || (int64_t)p.resp_first + p.n_resp > n_resp_total) return PBA_DESC_RESP_RANGE;
  int64_t e = (int64_t)p.start + p.prompt_len;
  for (int k = 0; k < p.n_resp; ++k) {
    const int r = resp_len[p.resp_first + k];
    if (r < 0) return PBA_DESC_NEGATIVE;
    e += r;
  }
  if (e > S) return PBA_DESC_BOUNDS;
  return 0;
}

// Block 0: validates every pack, records the first offending one in every
// map's status word and clears the totals.  Pack i's order check needs pack
// i-1 to be valid, which holds whenever i is the first offender.
__device__ void validate(const pba_pack* __restrict__ packs, int n_packs, const int32_t* __restrict__ resp_len,
                         int n_resp_total, const MapSet& ms) {
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = 0x7fffffff;
  __syncthreads();
  for (int i = threadIdx.x; i < n_packs; i += kThreads) {
    int code = check_pack(packs, i, resp_len, n_resp_total, ms.B, ms.S);
    if (code == 0 && i > 0 && check_pack(packs, i - 1, resp_len, n_resp_total, ms.B, ms.S) == 0) {
      const pba_pack a = packs[i - 1], b = packs[i];
      if (b.row < a.row || (b.row == a.row && (int64_t)b.start < pack_end(a, resp_len))) code = PBA_DESC_ORDER;
    }
    if (code != 0) atomicMin(&first_bad, i);
  }
  __syncthreads();
  if (threadIdx.x < ms.n) {
    const MapOut& m = ms.m[threadIdx.x];
    const int i = first_bad;
    if (i == 0x7fffffff) {
      m.status[0] = PBA_DESC_OK;
      m.status[1] = -1;
    } else {
      const int code = check_pack(packs, i, resp_len, n_resp_total, ms.B, ms.S);
      m.status[0] = code ? code : PBA_DESC_ORDER;
      m.status[1] = i;
    }
    m.totals[0] = m.totals[1] = m.totals[2] = 0;
  }
}

// Blocks 1..: one thread per token.  Locates its pack by binary search over
// the descriptors, then its branch, then its windows.  Only in-bounds reads
// even for invalid descriptors.
__global__ void __launch_bounds__(kThreads) map_tokens(const pba_pack* __restrict__ packs, int n_packs,
                                                       const int32_t* __restrict__ resp_len, int n_resp_total,
                                                       MapSet ms) {
  if (blockIdx.x == 0) {
    validate(packs, n_packs, resp_len, n_resp_total, ms);
    return;
  }
  const int64_t t = (int64_t)(blockIdx.x - 1) * kThreads + threadIdx.x;
  const int B = ms.B, S = ms.S;
  if (t >= (int64_t)B * S) return;
  const int b = (int)(t / S), s = (int)(t % S);
  // last pack with (row, start) <= (b, s)
  int lo = 0, hi = n_packs;  // answer in [lo-1, hi-1]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const pba_pack p = packs[mid];
    if (p.row < b || (p.row == b && p.start <= s)) lo = mid + 1; else hi = mid;
  }
  int pk = -1, br = 0;
  int kv_lo = s + 1, pre_lo = 0, pre_hi = 0, q_end = s;
  if (lo > 0) {
    const int pi = lo - 1;
    const pba_pack p = packs[pi];
    const bool sane = p.row == b && p.prompt_len >= 0 && p.n_resp >= 0 && p.resp_first >= 0 &&
                      (int64_t)p.resp_first + p.n_resp <= n_resp_total;
    if (sane) {
      const int64_t pstart = p.start, pend_prompt = (int64_t)p.start + p.prompt_len;
      if (s < pend_prompt) {
        pk = pi;
        kv_lo = (int)pstart;
        int64_t e = pend_prompt;
        for (int k = 0; k < p.n_resp; ++k) e += resp_len[p.resp_first + k];
        q_end = (int)min(e, (int64_t)S);
      } else {
        int64_t pos = pend_prompt;
        for (int k = 0; k < p.n_resp; ++k) {
          const int64_t r = resp_len[p.resp_first + k];
          if (s < pos + r) {
            pk = pi;
            br = k + 1;
            q_end = (int)min(pos + r, (int64_t)S);
            if (p.prompt_len == 0) {
              kv_lo = (int)pos;            // no prompt: just the own run
            } else if (pos == pend_prompt) {
              kv_lo = (int)pstart;         // own run starts right after the prompt: one run
            } else {
              kv_lo = (int)pos;            // prompt run, gap (siblings), own run
              pre_lo = (int)pstart;
              pre_hi = (int)pend_prompt;
            }
            break;
          }
          pos += r;
        }
      }
    }
  }
  const int4 win = make_int4(kv_lo, pre_lo, pre_hi, q_end);
  for (int i = 0; i < ms.n; ++i) {
    ms.m[i].tok_pack[t] = pk;
    ms.m[i].tok_branch[t] = br;
    reinterpret_cast<int4*>(ms.m[i].tok_win)[t] = win;
  }
}

__device__ __forceinline__ int overlap(int a0, int a1, int b0, int b1) {
  const int lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
  return hi > lo ? hi - lo : 0;
}

// One block per (query tile, row, map): the tile's query windows go to LDS,
// then each thread counts the visible pairs of some key tiles exactly.
__global__ void __launch_bounds__(kThreads) map_classify(MapSet ms) {
  const MapOut& m = ms.m[blockIdx.z];
  if (m.status[0] != 0) return;
  const int qt = blockIdx.x, b = blockIdx.y;
  if (qt >= m.nqt) return;
  __shared__ int4 win[256];
  __shared__ int cnt[3];
  const int S = ms.S, bm = m.bm, bn = m.bn, nqt = m.nqt, nkt = m.nkt;
  const int q0 = qt * bm;
  if (threadIdx.x < 3) cnt[threadIdx.x] = 0;
  for (int r = threadIdx.x; r < bm; r += kThreads) {
    const int i = q0 + r;
    win[r] = i < S ? reinterpret_cast<const int4*>(m.tok_win)[(int64_t)b * S + i] : make_int4(i + 1, 0, 0, i);
  }
  __syncthreads();
  // Key tiles in chunks of up to 256; a chunk's rows are split among the
  // threads that the chunk leaves free (rc row slices per key tile), and the
  // slices' counts meet in LDS.
  __shared__ int tc[kThreads];
  int nf = 0, np = 0, ns = 0;
  for (int kc = 0; kc < nkt; kc += kThreads) {
    const int nk = min(nkt - kc, kThreads);
    const int rc = max(1, min(kThreads / nk, bm));
    for (int i = threadIdx.x; i < nk; i += kThreads) tc[i] = 0;
    __syncthreads();
    if (threadIdx.x < nk * rc) {
      const int kl = threadIdx.x % nk, slice = threadIdx.x / nk;
      const int k0 = (kc + kl) * bn, k1 = k0 + bn;
      int c = 0;
      for (int r = slice * bm / rc; r < (slice + 1) * bm / rc; ++r) {
        const int4 w = win[r];
        c += overlap(w.y, w.z, k0, k1) + overlap(w.x, q0 + r + 1, k0, k1);
      }
      atomicAdd(&tc[kl], c);
    }
    __syncthreads();
    for (int kl = threadIdx.x; kl < nk; kl += kThreads) {
      const int c = tc[kl];
      const int v = c == bm * bn ? PBA_TILE_FULL : (c == 0 ? PBA_TILE_SKIP : PBA_TILE_PARTIAL);
      m.cls[((int64_t)b * nqt + qt) * nkt + kc + kl] = (uint8_t)v;
      nf += v == PBA_TILE_FULL;
      np += v == PBA_TILE_PARTIAL;
      ns += v == PBA_TILE_SKIP;
    }
    __syncthreads();
  }
  if (nf) atomicAdd(&cnt[0], nf);
  if (np) atomicAdd(&cnt[1], np);
  if (ns) atomicAdd(&cnt[2], ns);
  __syncthreads();
  if (threadIdx.x < 3 && cnt[threadIdx.x])
    atomicAdd((unsigned long long*)&m.totals[threadIdx.x], (unsigned long long)cnt[threadIdx.x]);
}

// One wave per list, lists of all maps numbered consecutively: per map,
// B*nqt query-tile lists (q2k), then B*nkt key-tile lists (k2q).  Stream
// compaction with ballots keeps ascending order.
__global__ void __launch_bounds__(kThreads) map_lists(MapSet ms) {
  const int lane = threadIdx.x & 63;
  int64_t list = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  int mi = 0;
  for (; mi < ms.n; ++mi) {
    const int64_t nl = (int64_t)ms.B * (ms.m[mi].nqt + ms.m[mi].nkt);
    if (list < nl) break;
    list -= nl;
  }
  if (mi >= ms.n) return;
  const MapOut& m = ms.m[mi];
  if (m.status[0] != 0) return;
  const int B = ms.B, nqt = m.nqt, nkt = m.nkt;
  const int64_t nq = (int64_t)B * nqt;
  const bool qmajor = list < nq;
  int n, b, t;
  int32_t *cnt, *idx;
  if (qmajor) {
    b = (int)(list / nqt); t = (int)(list % nqt); n = nkt;
    cnt = m.q2k_cnt + list * 2; idx = m.q2k_idx + list * nkt;
  } else {
    const int64_t l2 = list - nq;
    b = (int)(l2 / nkt); t = (int)(l2 % nkt); n = nqt;
    cnt = m.k2q_cnt + l2 * 2; idx = m.k2q_idx + l2 * nqt;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int written = 0, nfull = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int want = pass == 0 ? PBA_TILE_FULL : PBA_TILE_PARTIAL;
    for (int base = 0; base < n; base += 64) {
      const int e = base + lane;
      int v = PBA_TILE_SKIP;
      if (e < n) v = qmajor ? m.cls[((int64_t)b * nqt + t) * nkt + e] : m.cls[((int64_t)b * nqt + e) * nkt + t];
      const uint64_t msk = __ballot(v == want);
      if (v == want) idx[written + __popcll(msk & below)] = e;
      written += __popcll(msk);
    }
    if (pass == 0) nfull = written;
  }
  for (int e = written + lane; e < n; e += 64) idx[e] = -1;
  if (lane == 0) {
    cnt[0] = nfull;
    cnt[1] = written - nfull;
  }
}

// Work order of one side of one map: the tiles sorted by visit count
// (n_full + n_partial), descending, ties by index ascending.  Up to
// kOrderLds tiles: a bitonic sort in LDS of unique keys that encode both
// (so the result is the same as a stable sort).  Beyond that: a stable
// counting sort through the map's work area (histogram, scan from the
// largest count down, then placement one chunk at a time), accessed with
// device-scope atomics only.
__global__ void __launch_bounds__(kOrderThreads) map_order(MapSet ms) {
  const MapOut& m = ms.m[blockIdx.y];
  if (m.status[0] != 0) return;
  __shared__ int s_c[kOrderLds];
  __shared__ int s_sum[kOrderThreads];
  const int tid = threadIdx.x;
  const bool qside = blockIdx.x == 0;
  const int B = ms.B, nqt = m.nqt, nkt = m.nkt;
  const int n = qside ? B * nqt : B * nkt;
  const int maxc = qside ? nkt : nqt;
  const int32_t* cnt = qside ? m.q2k_cnt : m.k2q_cnt;
  int32_t* order = qside ? m.q_order : m.k_order;
  auto count_of = [&](int i) { return min(max(cnt[2 * i] + cnt[2 * i + 1], 0), maxc); };

  if (n <= kOrderLds) {
    // Bitonic sort in LDS of the unique keys (maxc - count) * 2^11 + index
    // (count descending, index ascending; maxc < 2^19 and n <= 2^11, so the
    // keys fit in 31 bits), padded to a power of two with the largest int.
    int n2 = 1;
    while (n2 < n) n2 <<= 1;
    for (int i = tid; i < n2; i += kOrderThreads) s_c[i] = i < n ? ((maxc - count_of(i)) << 11) | i : 0x7fffffff;
    __syncthreads();
    for (int k = 2; k <= n2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += kOrderThreads) {
          const int l = i ^ j;
          if (l > i) {
            const int a = s_c[i], b = s_c[l];
            if ((a > b) == ((i & k) == 0)) {
              s_c[i] = b;
              s_c[l] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < n; i += kOrderThreads) order[i] = s_c[i] & 2047;
    return;
  }

  int32_t* hist = m.work + (qside ? 0 : nkt + 1);
  auto ld = [](int32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto st = [](int32_t* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  for (int c = tid; c <= maxc; c += kOrderThreads) st(hist + c, 0);
  __threadfence();
  __syncthreads();
  for (int i = tid; i < n; i += kOrderThreads) atomicAdd(hist + count_of(i), 1);
  __threadfence();
  __syncthreads();
  // Bucket starts: start[c] = number of tiles with a larger count.
  int running = 0;
  for (int top = maxc; top >= 0; top -= kOrderThreads) {
    const int c = top - tid;
    const int v = c >= 0 ? ld(hist + c) : 0;
    s_sum[tid] = v;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off <<= 1) {  // inclusive scan over tid
      const int x = tid >= off ? s_sum[tid - off] : 0;
      __syncthreads();
      s_sum[tid] += x;
      __syncthreads();
    }
    if (c >= 0) st(hist + c, running + s_sum[tid] - v);
    running += s_sum[kOrderThreads - 1];
    __syncthreads();
  }
  __threadfence();
  __syncthreads();
  for (int base = 0; base < n; base += kOrderThreads) {
    const int i = base + tid;
    const int c = i < n ? count_of(i) : -1;
    s_c[tid] = c;
    __syncthreads();
    int before = 0;
    bool last = true;
    for (int t = 0; t < kOrderThreads; ++t) {
      const int x = s_c[t];
      before += (t < tid && x == c) ? 1 : 0;
      last = last && !(t > tid && x == c);
    }
    int start = 0;
    if (i < n) {
      start = ld(hist + c);
      order[start + before] = i;
    }
    __threadfence();
    __syncthreads();
    if (i < n && last) st(hist + c, start + before + 1);
    __threadfence();
    __syncthreads();
  }
}

// Aligned positions and log-prob gather rows from the per-token windows
// ("DPO Preference Packing: Dense Masks and Sparse Execution", section
// "Layout requirements": a response token keeps the position and the
// predicting row it has in its own [prompt | response] sequence, so a
// response's first token reads the last prompt row; "Pack training sequences
// to reduce padding waste": positions restart and no target crosses an
// example boundary).  Token s sees [pre_lo, pre_hi) U [kv_lo, s]: its
// sequence so far is the prompt run (if separate) then [kv_lo, s], so its
// position is (pre_hi - pre_lo) + (s - kv_lo) and its predecessor s - 1
// inside [kv_lo, s], else pre_hi - 1, else none.  One thread per token.
__global__ void __launch_bounds__(kThreads) map_positions(PosArgs a) {
  if (a.status[0] != 0) return;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= a.ntok) return;
  const int s = (int)(t % a.S);
  const int br = a.tok_branch[t];
  const int4 w = reinterpret_cast<const int4*>(a.tok_win)[t];
  const bool pad = a.tok_pack[t] < 0;
  const int pre = w.z - w.y;
  const int pos = pad ? 0 : pre + (s - w.x);
  const int src = pad ? -1 : (s > w.x ? s - 1 : (pre > 0 ? w.z - 1 : -1));
  if (a.pos) a.pos[t] = pos;
  if (a.src) a.src[t] = src;
  if (a.mask) a.mask[t] = (uint8_t)(br > 0 && src >= 0);
}

}  // namespace

hipError_t launch_positions(const PosArgs& a, hipStream_t stream) {
  if (a.ntok <= 0) return hipSuccess;
  map_positions<<<(unsigned)((a.ntok + kThreads - 1) / kThreads), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_maps(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                       const pba_block_map* maps, int n_maps, hipStream_t stream) {
  MapSet ms;
  ms.n = n_maps;
  ms.B = maps[0].B;
  ms.S = maps[0].S;
  int max_nqt = 1;
  int64_t lists = 0;
  for (int i = 0; i < n_maps; ++i) {
    const pba_block_map& s = maps[i];
    MapOut& o = ms.m[i];
    o.bm = s.block_m; o.bn = s.block_n; o.nqt = s.nqt; o.nkt = s.nkt;
    o.tok_pack = s.tok_pack; o.tok_branch = s.tok_branch; o.tok_win = s.tok_win; o.cls = s.cls;
    o.q2k_cnt = s.q2k_cnt; o.q2k_idx = s.q2k_idx; o.k2q_cnt = s.k2q_cnt; o.k2q_idx = s.k2q_idx;
    o.totals = s.totals; o.status = s.status; o.q_order = s.q_order; o.k_order = s.k_order; o.work = s.work;
    max_nqt = max(max_nqt, s.nqt);
    lists += (int64_t)ms.B * (s.nqt + s.nkt);
  }
  const int64_t ntok = (int64_t)ms.B * ms.S;
  map_tokens<<<(unsigned)(1 + (ntok + kThreads - 1) / kThreads), kThreads, 0, stream>>>(packs, n_packs, resp_len,
                                                                                       n_resp_total, ms);
  map_classify<<<dim3(max_nqt, ms.B, n_maps), kThreads, 0, stream>>>(ms);
  map_lists<<<(unsigned)((lists + 3) / 4), kThreads, 0, stream>>>(ms);
  map_order<<<dim3(2, n_maps), kOrderThreads, 0, stream>>>(ms);
  return hipGetLastError();
}

}  // namespace pba
