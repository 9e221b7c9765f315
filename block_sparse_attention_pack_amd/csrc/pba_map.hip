// Block map kernels: descriptor checks, per-token ids and windows, tile
// classification, visit lists.  Integer work only; results are bit-exact.
//
// The mask being summarised is the branch-aware, pack-bounded causal mask
// ("DPO Preference Packing: Dense Masks and Sparse Execution", section
// "Layout requirements"; pack boundaries as in "Pack training sequences to
// reduce padding waste", section "Preserve attention boundaries").  For a
// query i the visible keys are at most two runs, [pre_lo, pre_hi) (the
// prompt, seen from a later response) and [kv_lo, i]; a key j is seen by
// the queries [j, q_end).  Tiles with no visible pair are skipped, as a
// block mask skips fully masked blocks (same page, section "Dense and sparse
// execution").
#include "pba_internal.h"

namespace pba {
namespace {

constexpr int kThreads = 256;

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

// One block: validates every pack, records the first offending one, and
// clears the totals.  Pack i's order check needs pack i-1 to be valid,
// which holds whenever i is the first offender.
__global__ void __launch_bounds__(kThreads) map_validate(const pba_pack* __restrict__ packs, int n_packs,
                                                         const int32_t* __restrict__ resp_len, int n_resp_total,
                                                         int B, int S, int32_t* status, int64_t* totals) {
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = 0x7fffffff;
  __syncthreads();
  for (int i = threadIdx.x; i < n_packs; i += kThreads) {
    int code = check_pack(packs, i, resp_len, n_resp_total, B, S);
    if (code == 0 && i > 0 && check_pack(packs, i - 1, resp_len, n_resp_total, B, S) == 0) {
      const pba_pack a = packs[i - 1], b = packs[i];
      if (b.row < a.row || (b.row == a.row && (int64_t)b.start < pack_end(a, resp_len))) code = PBA_DESC_ORDER;
    }
    if (code != 0) atomicMin(&first_bad, i);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int i = first_bad;
    if (i == 0x7fffffff) {
      status[0] = PBA_DESC_OK;
      status[1] = -1;
    } else {
      int code = check_pack(packs, i, resp_len, n_resp_total, B, S);
      status[0] = code ? code : PBA_DESC_ORDER;
      status[1] = i;
    }
    totals[0] = totals[1] = totals[2] = 0;
  }
}

// One thread per token: locate its pack by binary search over the sorted
// descriptors, then its branch, then its windows.
__global__ void __launch_bounds__(kThreads) map_tokens(const pba_pack* __restrict__ packs, int n_packs,
                                                       const int32_t* __restrict__ resp_len, int B, int S,
                                                       const int32_t* __restrict__ status, int32_t* tok_pack,
                                                       int32_t* tok_branch, int32_t* tok_win) {
  if (status[0] != 0) return;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
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
    if (p.row == b) {
      const int pstart = p.start, pend_prompt = p.start + p.prompt_len;
      int pos = pend_prompt;
      if (s < pend_prompt) {
        pk = pi;
        br = 0;
        kv_lo = pstart;
        q_end = (int)pack_end(p, resp_len);
      } else {
        for (int k = 0; k < p.n_resp; ++k) {
          const int r = resp_len[p.resp_first + k];
          if (s < pos + r) {
            pk = pi;
            br = k + 1;
            q_end = pos + r;
            if (p.prompt_len == 0) {
              kv_lo = pos;                 // no prompt: just the own run
            } else if (pos == pend_prompt) {
              kv_lo = pstart;              // own run starts right after the prompt: one run
            } else {
              kv_lo = pos;                 // prompt run, gap (siblings), own run
              pre_lo = pstart;
              pre_hi = pend_prompt;
            }
            break;
          }
          pos += r;
        }
      }
    }
  }
  tok_pack[t] = pk;
  tok_branch[t] = br;
  reinterpret_cast<int4*>(tok_win)[t] = make_int4(kv_lo, pre_lo, pre_hi, q_end);
}

__device__ __forceinline__ int overlap(int a0, int a1, int b0, int b1) {
  const int lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
  return hi > lo ? hi - lo : 0;
}

// One block per (query tile, row): the tile's query windows go to LDS, then
// each thread counts the visible pairs of some key tiles exactly.
__global__ void __launch_bounds__(kThreads) map_classify(const int32_t* __restrict__ tok_win, int S, int bm, int bn,
                                                         int nqt, int nkt, const int32_t* __restrict__ status,
                                                         uint8_t* cls, int64_t* totals) {
  if (status[0] != 0) return;
  __shared__ int4 win[256];
  __shared__ int cnt[3];
  const int qt = blockIdx.x, b = blockIdx.y;
  const int q0 = qt * bm;
  if (threadIdx.x < 3) cnt[threadIdx.x] = 0;
  for (int r = threadIdx.x; r < bm; r += kThreads) {
    const int i = q0 + r;
    win[r] = i < S ? reinterpret_cast<const int4*>(tok_win)[(int64_t)b * S + i] : make_int4(i + 1, 0, 0, i);
  }
  __syncthreads();
  int nf = 0, np = 0, ns = 0;
  for (int kt = threadIdx.x; kt < nkt; kt += kThreads) {
    const int k0 = kt * bn, k1 = k0 + bn;
    int c = 0;
    for (int r = 0; r < bm; ++r) {
      const int4 w = win[r];
      c += overlap(w.y, w.z, k0, k1) + overlap(w.x, q0 + r + 1, k0, k1);
    }
    const int v = c == bm * bn ? PBA_TILE_FULL : (c == 0 ? PBA_TILE_SKIP : PBA_TILE_PARTIAL);
    cls[((int64_t)b * nqt + qt) * nkt + kt] = (uint8_t)v;
    nf += v == PBA_TILE_FULL;
    np += v == PBA_TILE_PARTIAL;
    ns += v == PBA_TILE_SKIP;
  }
  if (nf) atomicAdd(&cnt[0], nf);
  if (np) atomicAdd(&cnt[1], np);
  if (ns) atomicAdd(&cnt[2], ns);
  __syncthreads();
  if (threadIdx.x < 3 && cnt[threadIdx.x]) atomicAdd((unsigned long long*)&totals[threadIdx.x], (unsigned long long)cnt[threadIdx.x]);
}

// One wave per list.  Lists 0 .. B*nqt-1 are query tiles (q2k), the rest key
// tiles (k2q).  Stream compaction with ballots keeps ascending order.
__global__ void __launch_bounds__(kThreads) map_lists(const uint8_t* __restrict__ cls, int B, int nqt, int nkt,
                                                      const int32_t* __restrict__ status, int32_t* q2k_cnt,
                                                      int32_t* q2k_idx, int32_t* k2q_cnt, int32_t* k2q_idx) {
  if (status[0] != 0) return;
  const int lane = threadIdx.x & 63;
  const int64_t list = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nq = (int64_t)B * nqt, total = nq + (int64_t)B * nkt;
  if (list >= total) return;
  const bool qmajor = list < nq;
  int n, b, t;
  int32_t *cnt, *idx;
  if (qmajor) {
    b = (int)(list / nqt); t = (int)(list % nqt); n = nkt;
    cnt = q2k_cnt + list * 2; idx = q2k_idx + list * nkt;
  } else {
    const int64_t l2 = list - nq;
    b = (int)(l2 / nkt); t = (int)(l2 % nkt); n = nqt;
    cnt = k2q_cnt + l2 * 2; idx = k2q_idx + l2 * nqt;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int written = 0, nfull = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int want = pass == 0 ? PBA_TILE_FULL : PBA_TILE_PARTIAL;
    for (int base = 0; base < n; base += 64) {
      const int e = base + lane;
      int v = PBA_TILE_SKIP;
      if (e < n) v = qmajor ? cls[((int64_t)b * nqt + t) * nkt + e] : cls[((int64_t)b * nqt + e) * nkt + t];
      const uint64_t m = __ballot(v == want);
      if (v == want) idx[written + __popcll(m & below)] = e;
      written += __popcll(m);
    }
    if (pass == 0) nfull = written;
  }
  for (int e = written + lane; e < n; e += 64) idx[e] = -1;
  if (lane == 0) {
    cnt[0] = nfull;
    cnt[1] = written - nfull;
  }
}


// One block per order array (block 0: query tiles, block 1: key tiles).
// Stable counting sort by visit count, descending: a histogram of the
// counts, its exclusive scan from the largest count down (bucket starts),
// then placement in index order, one chunk of kThreads items at a time,
// each item going after the earlier items of its bucket.  The histogram
// lives in map->work and is accessed with device-scope atomics only, so
// every phase sees the previous one's values in L2.
__global__ void __launch_bounds__(kThreads) map_order(int B, int nqt, int nkt, const int32_t* __restrict__ status,
                                                      const int32_t* __restrict__ q2k_cnt,
                                                      const int32_t* __restrict__ k2q_cnt, int32_t* q_order,
                                                      int32_t* k_order, int32_t* work) {
  if (status[0] != 0) return;
  __shared__ int s_c[kThreads];
  __shared__ int s_sum[kThreads];
  const int tid = threadIdx.x;
  const bool qside = blockIdx.x == 0;
  const int n = qside ? B * nqt : B * nkt;
  const int maxc = qside ? nkt : nqt;
  const int32_t* cnt = qside ? q2k_cnt : k2q_cnt;
  int32_t* order = qside ? q_order : k_order;
  int32_t* hist = work + (qside ? 0 : nkt + 1);
  auto ld = [](int32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto st = [](int32_t* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  auto count_of = [&](int i) { return min(max(cnt[2 * i] + cnt[2 * i + 1], 0), maxc); };

  for (int c = tid; c <= maxc; c += kThreads) st(hist + c, 0);
  __threadfence();
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) atomicAdd(hist + count_of(i), 1);
  __threadfence();
  __syncthreads();
  // Bucket starts: start[c] = number of items with a larger count.
  int running = 0;
  for (int top = maxc; top >= 0; top -= kThreads) {
    const int c = top - tid;
    const int v = c >= 0 ? ld(hist + c) : 0;
    s_sum[tid] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan over tid
      const int x = tid >= off ? s_sum[tid - off] : 0;
      __syncthreads();
      s_sum[tid] += x;
      __syncthreads();
    }
    if (c >= 0) st(hist + c, running + s_sum[tid] - v);
    running += s_sum[kThreads - 1];
    __syncthreads();
  }
  __threadfence();
  __syncthreads();
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    const int c = i < n ? count_of(i) : -1;
    s_c[tid] = c;
    __syncthreads();
    int before = 0;
    bool last = true;
    for (int t = 0; t < kThreads; ++t) {
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

}  // namespace

hipError_t launch_map(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                      const pba_block_map& m, hipStream_t stream) {
  map_validate<<<1, kThreads, 0, stream>>>(packs, n_packs, resp_len, n_resp_total, m.B, m.S, m.status, m.totals);
  const int64_t ntok = (int64_t)m.B * m.S;
  map_tokens<<<(unsigned)((ntok + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
      packs, n_packs, resp_len, m.B, m.S, m.status, m.tok_pack, m.tok_branch, m.tok_win);
  map_classify<<<dim3(m.nqt, m.B), kThreads, 0, stream>>>(m.tok_win, m.S, m.block_m, m.block_n, m.nqt, m.nkt,
                                                          m.status, m.cls, m.totals);
  const int64_t lists = (int64_t)m.B * (m.nqt + m.nkt);
  map_lists<<<(unsigned)((lists + 3) / 4), kThreads, 0, stream>>>(m.cls, m.B, m.nqt, m.nkt, m.status, m.q2k_cnt,
                                                                 m.q2k_idx, m.k2q_cnt, m.k2q_idx);
  map_order<<<2, kThreads, 0, stream>>>(m.B, m.nqt, m.nkt, m.status, m.q2k_cnt, m.k2q_cnt, m.q_order, m.k_order,
                                        m.work);
  return hipGetLastError();
}

}  // namespace pba
