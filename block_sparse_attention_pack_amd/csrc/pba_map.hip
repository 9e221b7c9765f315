// Block map kernels: descriptor checks, per-token ids and windows, tile
// classification, visit lists, work orders.  Integer work only; results are
// bit-exact.  Several maps of the same rows (different tile shapes) are built
// together: each stage is one launch covering all of them (two launches in
// all, three when a side has more than 2048 tiles).
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
//   map_tiles     one wave per visit list: classifies each tile of its
//                 row (q2k, from the query windows) or column (k2q, from the
//                 key runs) with two ballots, writes the full then the
//                 partial tiles; the last block to finish one side of one
//                 map sorts that side's work order by rank in LDS and sums
//                 the map's totals
//   map_order     only for sides of more than 2048 tiles: a stable counting
//                 sort through the work area
//   map_positions (its own entry point, on a built map) aligned position
//                 ids, log-prob gather rows and the response loss mask
#include "pba_next.h"

namespace pba {
namespace {

constexpr int kThreads = 256;
constexpr int kOrderThreads = 1024;
constexpr int kOrderLds = 2048;  // tiles per side sorted in LDS; more use the chunked path
constexpr int kTilesThreads = 512;
constexpr int kTilesWaves = kTilesThreads / 64;  // lists per map_tiles block

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
    m.work[m.nqt + m.nkt + 2] = 0;  // map_tiles arrival counters (query side, key side)
    m.work[m.nqt + m.nkt + 3] = 0;
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

// Lists of all maps numbered consecutively: per map, B*nqt query-tile lists
// (q2k), then B*nkt key-tile lists (k2q).  A group is the lists of one side
// of one map; its arrival counter sits in the map's work area.
__device__ __forceinline__ int64_t group_begin(const MapSet& ms, int g) {
  int64_t o = 0;
  for (int i = 0; i < g; ++i) {
    const MapOut& m = ms.m[i >> 1];
    o += (int64_t)ms.B * ((i & 1) ? m.nkt : m.nqt);
  }
  return o;
}

__device__ __forceinline__ int32_t* group_counter(const MapOut& m, bool qside) {
  return m.work + m.nqt + m.nkt + (qside ? 2 : 3);
}

// Stable rank sort of one side's tiles by visit count, descending, ties by
// index ascending, for up to kOrderLds tiles: the keys
// (maxc - count) * 2^11 + index are unique, and a tile's place is the
// number of smaller keys.  The whole block takes part; when there are fewer
// tiles than threads, several threads share one tile's count, each over a
// slice of the keys, and their counts meet in LDS.
__device__ void rank_order(const int32_t* cnt, int n, int maxc, int32_t* order, int* s_key, int* s_rank) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int n4 = (n + 3) & ~3, nv = n4 >> 2;
  for (int i = tid; i < n4; i += nt) {
    int key = 0x7fffffff;
    if (i < n) key = ((maxc - min(max(cnt[2 * i] + cnt[2 * i + 1], 0), maxc)) << 11) | i;
    s_key[i] = key;
    s_rank[i] = 0;
  }
  __syncthreads();
  const int parts = max(1, min(8, nt / n));
  const int4* kv = reinterpret_cast<const int4*>(s_key);
  for (int x = tid; x < n * parts; x += nt) {
    const int i = x / parts, p = x % parts;
    const int key = s_key[i];
    const int j0 = p * nv / parts, j1 = (p + 1) * nv / parts;
    int rank = 0;
#pragma unroll 8
    for (int j = j0; j < j1; ++j) {
      const int4 k4 = kv[j];
      rank += (k4.x < key) + (k4.y < key) + (k4.z < key) + (k4.w < key);
    }
    if (parts == 1) s_rank[i] = rank;
    else atomicAdd(&s_rank[i], rank);
  }
  __syncthreads();
  for (int i = tid; i < n; i += nt) order[s_rank[i]] = i;
  __syncthreads();
}

// Totals of one map from its query-tile counts: n_full, n_partial, and the
// remaining tile pairs as n_skip.
__device__ void map_totals(const MapOut& m, int B, int64_t* s_red) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int n = B * m.nqt;
  int64_t f = 0, p = 0;
  for (int i = tid; i < n; i += nt) {
    f += m.q2k_cnt[2 * i];
    p += m.q2k_cnt[2 * i + 1];
  }
  s_red[tid] = f;
  s_red[nt + tid] = p;
  __syncthreads();
  for (int off = nt >> 1; off > 0; off >>= 1) {
    if (tid < off) {
      s_red[tid] += s_red[tid + off];
      s_red[nt + tid] += s_red[nt + tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int64_t all = (int64_t)B * m.nqt * m.nkt;
    m.totals[0] = s_red[0];
    m.totals[1] = s_red[nt];
    m.totals[2] = all - s_red[0] - s_red[nt];
  }
  __syncthreads();
}

// One wave per list, one lane per tile of the list (64 tiles at a time).
// For a q2k list the windows of the tile row's queries go to LDS (row i
// sees [pre_lo, pre_hi) and [kv_lo, i]) and a lane counts its tile's
// visible pairs row by row.  For a k2q list the key runs of the column's
// keys (key j is seen by the queries [j, q_end)) reduce to a prefix maximum
// and a minimum of the run ends, which decide each query tile in O(1).  Both
// sides decide from the exact visible pairs, so both agree.  The full
// tiles are written in ascending order by ballot compaction, then the
// partial ones (classes recomputed for lists of more than 64 tiles), then -1
// fill and the counts; q2k waves also write the classes.  The last block to finish a group (all lists of one side of one
// map) sorts that side's work order and, for the query side, sums the map's
// totals; sides of more than kOrderLds tiles are left to map_order.
__global__ void __launch_bounds__(kTilesThreads) map_tiles(MapSet ms) {
  __shared__ __attribute__((aligned(16))) int s_key[kOrderLds];
  __shared__ int s_rank[kOrderLds];
  __shared__ int64_t s_red[2 * kTilesThreads];
  __shared__ int4 s_win[kTilesWaves][256];
  __shared__ int s_last[2 * kMaxMapsPerBuild];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int B = ms.B, S = ms.S;
  const int64_t first = (int64_t)blockIdx.x * kTilesWaves;
  int64_t list = first + w;
  int mi = 0;
  for (; mi < ms.n; ++mi) {
    const int64_t nl = (int64_t)B * (ms.m[mi].nqt + ms.m[mi].nkt);
    if (list < nl) break;
    list -= nl;
  }
  const bool active = mi < ms.n && ms.m[mi].status[0] == 0;
  const MapOut& m = ms.m[active ? mi : 0];
  const int nqt = m.nqt, nkt = m.nkt;
  const int64_t nq = (int64_t)B * nqt;
  const bool qmajor = list < nq;
  int n = 0, b = 0, t = 0;
  int32_t *cnt = nullptr, *idx = nullptr;
  if (active) {
    if (qmajor) {
      b = (int)(list / nqt); t = (int)(list % nqt); n = nkt;
      cnt = m.q2k_cnt + list * 2; idx = m.q2k_idx + list * nkt;
    } else {
      const int64_t l2 = list - nq;
      b = (int)(l2 / nkt); t = (int)(l2 % nkt); n = nqt;
      cnt = m.k2q_cnt + l2 * 2; idx = m.k2q_idx + l2 * nqt;
    }
  }
  const int nunit = qmajor ? m.bm : m.bn, ext = qmajor ? m.bn : m.bm;
  const int u0 = t * nunit;  // first row (q2k) or key (k2q) of the tile row / column
  int4* win = s_win[w];
  int min_end = 0x7fffffff;  // k2q: smallest run end over the tile's keys
  if (active) {
    if (qmajor) {
      for (int r = lane; r < nunit; r += 64) {
        const int i = u0 + r;
        // Positions >= S are pad: no visible run.
        win[r] = i < S ? reinterpret_cast<const int4*>(m.tok_win)[(int64_t)b * S + i] : make_int4(i + 1, 0, 0, i);
      }
    } else {
      // Key u0 + r is seen by the queries [u0 + r, q_end) (empty for pad and
      // keys >= S).  Lane l holds keys 4l .. 4l+3; win[r].x becomes the
      // largest run end over the non-empty runs of keys u0 .. u0 + r
      // (INT_MIN if none), by a wave scan.
      int e4[4], pm = (int)0x80000000;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * lane + u, i = u0 + r;
        const int qe = (r < nunit && i < S) ? reinterpret_cast<const int4*>(m.tok_win)[(int64_t)b * S + i].w : i;
        if (r < nunit) min_end = min(min_end, qe);
        pm = max(pm, qe > i ? qe : (int)0x80000000);
        e4[u] = pm;
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(pm, off);
        if (lane >= off) pm = max(pm, o);
      }
      const int before = __shfl_up(pm, 1);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * lane + u;
        if (r < nunit) win[r].x = lane ? max(before, e4[u]) : e4[u];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) min_end = min(min_end, __shfl_xor(min_end, off));
    }
  }
  __syncthreads();
  if (active) {
    // Class of tile e: exact count per unit against [e*ext, (e+1)*ext).
    auto classify = [&](int e) -> int {
      if (e >= n) return PBA_TILE_SKIP;
      const int lo = e * ext, hi = lo + ext;
      bool all_full = true, any_hit = false;
      if (qmajor) {
#pragma unroll 4
        for (int r = 0; r < nunit; ++r) {
          const int4 v = win[r];
          const int c = overlap(v.y, v.z, lo, hi) + overlap(v.x, u0 + r + 1, lo, hi);
          all_full = all_full && c == ext;
          any_hit = any_hit || c > 0;
        }
      } else {
        // Every pair visible iff every key precedes the first query and
        // every key's run reaches the last one; some pair visible iff a key
        // below hi has a non-empty run ending after lo (a run starts at its
        // key, so a key in [lo, hi) with a non-empty run qualifies).
        all_full = u0 + nunit - 1 <= lo && min_end >= hi;
        any_hit = hi > u0 && win[min(hi - u0, nunit) - 1].x > lo;
      }
      return all_full ? PBA_TILE_FULL : (any_hit ? PBA_TILE_PARTIAL : PBA_TILE_SKIP);
    };
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int c0 = PBA_TILE_SKIP, written = 0, npart = 0;
    for (int base = 0; base < n; base += 64) {
      const int e = base + lane;
      const int c = classify(e);
      if (base == 0) c0 = c;
      if (qmajor && e < n) m.cls[((int64_t)b * nqt + t) * nkt + e] = (uint8_t)c;
      const uint64_t mf = __ballot(c == PBA_TILE_FULL);
      if (c == PBA_TILE_FULL) idx[written + __popcll(mf & below)] = e;
      written += __popcll(mf);
      npart += __popcll(__ballot(c == PBA_TILE_PARTIAL));
    }
    const int nfull = written;
    for (int base = 0; npart > 0 && base < n; base += 64) {
      const int e = base + lane;
      const int c = base == 0 ? c0 : classify(e);
      const uint64_t mp = __ballot(c == PBA_TILE_PARTIAL);
      if (c == PBA_TILE_PARTIAL) idx[written + __popcll(mp & below)] = e;
      written += __popcll(mp);
    }
    for (int e = written + lane; e < n; e += 64) idx[e] = -1;
    if (lane == 0) {
      cnt[0] = nfull;
      cnt[1] = written - nfull;
    }
  }
  // Arrival: every group this block's lists touch counts the block once.
  // Each wave waits until its own stores have reached the L2 (the barrier
  // alone does not wait for global stores), then one agent-scope release
  // (an L2 write-back, which covers every wave's stores) publishes them
  // before the counter moves, and the last arriver's acquire (L2
  // invalidate) comes before anything it reads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ng = 2 * ms.n;
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    bool any_last = false;
    for (int g = 0; g < ng; ++g) {
      const MapOut& mg = ms.m[g >> 1];
      const int64_t g0 = group_begin(ms, g), g1 = g0 + (int64_t)B * ((g & 1) ? mg.nkt : mg.nqt);
      int lastflag = 0;
      if (g0 < first + kTilesWaves && first < g1) {
        const int64_t nblk = (g1 - 1) / kTilesWaves - g0 / kTilesWaves + 1;
        const int old = __hip_atomic_fetch_add(group_counter(mg, (g & 1) == 0), 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        lastflag = (int64_t)old == nblk - 1;
      }
      s_last[g] = lastflag;
      any_last = any_last || lastflag;
    }
    if (any_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  for (int g = 0; g < ng; ++g) {
    if (!s_last[g]) continue;
    const MapOut& m = ms.m[g >> 1];
    if (m.status[0] != 0) continue;
    const bool qside = (g & 1) == 0;
    const int n = qside ? B * m.nqt : B * m.nkt;
    if (n <= kOrderLds)
      rank_order(qside ? m.q2k_cnt : m.k2q_cnt, n, qside ? m.nkt : m.nqt, qside ? m.q_order : m.k_order, s_key,
                 s_rank);
    if (qside) map_totals(m, B, s_red);
  }
}

// Work order of one side of one map with more than kOrderLds tiles (smaller
// sides are sorted by map_tiles): the tiles sorted by visit count
// (n_full + n_partial), descending, ties by index ascending, by a stable
// counting sort through the map's work area (histogram, scan from the
// largest count down, then placement one chunk at a time), accessed with
// device-scope atomics only.
__global__ void __launch_bounds__(kOrderThreads) map_order(MapSet ms) {
  const MapOut& m = ms.m[blockIdx.y];
  if (m.status[0] != 0) return;
  __shared__ int s_c[kOrderThreads];
  __shared__ int s_sum[kOrderThreads];
  const int tid = threadIdx.x;
  const bool qside = blockIdx.x == 0;
  const int B = ms.B, nqt = m.nqt, nkt = m.nkt;
  const int n = qside ? B * nqt : B * nkt;
  const int maxc = qside ? nkt : nqt;
  const int32_t* cnt = qside ? m.q2k_cnt : m.k2q_cnt;
  int32_t* order = qside ? m.q_order : m.k_order;
  auto count_of = [&](int i) { return min(max(cnt[2 * i] + cnt[2 * i + 1], 0), maxc); };

  if (n <= kOrderLds) return;  // sorted in LDS by map_tiles

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
  bool big_side = false;  // a side with more tiles than map_tiles sorts in LDS
  int64_t lists = 0;
  for (int i = 0; i < n_maps; ++i) {
    const pba_block_map& s = maps[i];
    MapOut& o = ms.m[i];
    o.bm = s.block_m; o.bn = s.block_n; o.nqt = s.nqt; o.nkt = s.nkt;
    o.tok_pack = s.tok_pack; o.tok_branch = s.tok_branch; o.tok_win = s.tok_win; o.cls = s.cls;
    o.q2k_cnt = s.q2k_cnt; o.q2k_idx = s.q2k_idx; o.k2q_cnt = s.k2q_cnt; o.k2q_idx = s.k2q_idx;
    o.totals = s.totals; o.status = s.status; o.q_order = s.q_order; o.k_order = s.k_order; o.work = s.work;
    big_side = big_side || (int64_t)ms.B * max(s.nqt, s.nkt) > kOrderLds;
    lists += (int64_t)ms.B * (s.nqt + s.nkt);
  }
  const int64_t ntok = (int64_t)ms.B * ms.S;
  map_tokens<<<(unsigned)(1 + (ntok + kThreads - 1) / kThreads), kThreads, 0, stream>>>(packs, n_packs, resp_len,
                                                                                       n_resp_total, ms);
  map_tiles<<<(unsigned)((lists + kTilesWaves - 1) / kTilesWaves), kTilesThreads, 0, stream>>>(ms);
  if (big_side) map_order<<<dim3(2, n_maps), kOrderThreads, 0, stream>>>(ms);
  return hipGetLastError();
}

}  // namespace pba
