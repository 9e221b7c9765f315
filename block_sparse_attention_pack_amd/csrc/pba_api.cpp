// C ABI entry points: argument checks, map buffer carving, kernel launches.
// Nothing here allocates or synchronises; all work goes to the caller's
// stream.  Descriptor contents are checked on the device by the map kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "pba_next.h"
#include "../../include/pba_measure.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxB = 65535;
constexpr int kMaxS = 1 << 22;
constexpr int kMaxHeads = 4096;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool tile_ok(int t) { return t == 16 || t == 32 || t == 64 || t == 128 || t == 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Field sizes of a map, in the order they are carved from the buffer.
struct MapLayout {
  size_t off[13];
  size_t total;
};

MapLayout map_layout(int B, int S, int bm, int bn) {
  const size_t nqt = (size_t)((S + bm - 1) / bm), nkt = (size_t)((S + bn - 1) / bn);
  const size_t ntok = (size_t)B * S;
  const size_t sizes[13] = {
      4 * ntok,               // tok_pack
      4 * ntok,               // tok_branch
      16 * ntok,              // tok_win
      (size_t)B * nqt * nkt,  // cls
      8 * (size_t)B * nqt,    // q2k_cnt
      4 * (size_t)B * nqt * nkt,  // q2k_idx
      8 * (size_t)B * nkt,    // k2q_cnt
      4 * (size_t)B * nkt * nqt,  // k2q_idx
      3 * 8,                  // totals
      2 * 4,                  // status
      4 * (size_t)B * nqt,    // q_order
      4 * (size_t)B * nkt,    // k_order
      4 * (nqt + nkt + 4),    // work (order histograms, arrival counters)
  };
  MapLayout L;
  size_t o = 0;
  for (int i = 0; i < 13; ++i) {
    L.off[i] = o;
    o += align_up(sizes[i]);
  }
  L.total = o;
  return L;
}

// gfx950 check, cached per device.
int device_ok() {
  static std::mutex mu;
  static int cache[64];
  static bool init = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PBA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(mu);
  if (!init) {
    for (int i = 0; i < 64; ++i) cache[i] = 0;
    init = true;
  }
  if (cache[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return PBA_ERR_DEVICE;
    cache[dev] = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return cache[dev] == 1 ? PBA_OK : PBA_ERR_DEVICE;
}

int check_map(const pba_block_map* m, int B, int S, int bm, int bn) {
  if (!m || !m->tok_win || !m->q2k_cnt || !m->q2k_idx || !m->k2q_cnt || !m->k2q_idx || !m->status || !m->q_order ||
      !m->k_order || !m->totals)
    return PBA_ERR_NULL;
  if (m->B != B || m->S != S) return PBA_ERR_MAP;
  if (m->block_m != bm || m->block_n != bn) return PBA_ERR_TILE;
  if (m->nqt != (S + bm - 1) / bm || m->nkt != (S + bn - 1) / bn) return PBA_ERR_MAP;
  return PBA_OK;
}

int check_heads(int B, int S, int Hq, int Hkv, int D) {
  if (B < 1 || B > kMaxB || S < 1 || S > kMaxS || Hq < 1 || Hkv < 1 || Hq > kMaxHeads) return PBA_ERR_SHAPE;
  if (Hq % Hkv != 0) return PBA_ERR_HEADS;
  if (D != 64 && D != 128) return PBA_ERR_HEAD_DIM;
  return PBA_OK;
}

size_t bwd_scratch_bytes(int B, int S, int Hq, int D, size_t pairs);

// Split key tiles of bwd_dkdv: at most this many (position, kv group)
// pairs have a partial-sum area in the workspace.
size_t split_pairs(int B, int S, int Hq) {
  const size_t nkt = (size_t)((S + pba::kBwdBN - 1) / pba::kBwdBN);
  return std::min((size_t)pba::kMaxSplitPairs, (size_t)B * nkt * Hq);
}

// Workgroup slots per kv group for the split rule of bwd_dkdv when set by
// pba_set_bwd_split_slots (0: the device's compute units / Hkv).
std::atomic<int> g_split_slots{0};

// Compute units of the current device, cached per device (0 if unknown).
int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// The softmax is evaluated as exp2(s * scale * log2(e) - m) with the row
// maximum taken before scaling, which needs a positive, finite scale.
int check_scale(float scale) {
  return (scale > 0.f && scale < 3.0e38f) ? PBA_OK : PBA_ERR_SCALE;
}

// Tiles are read through buffer resources with 32-bit byte offsets: one
// batch row of the widest tensor ([S, Hq, D] bf16) must stay below 2 GiB.
int check_row_bytes(int S, int Hq, int D) {
  return (int64_t)S * Hq * D * 2 < ((int64_t)1 << 31) ? PBA_OK : PBA_ERR_SHAPE;
}

pba::MapView view_of(const pba_block_map* m) {
  pba::MapView v;
  v.B = m->B; v.S = m->S; v.bm = m->block_m; v.bn = m->block_n; v.nqt = m->nqt; v.nkt = m->nkt;
  v.tok_win = m->tok_win; v.q2k_cnt = m->q2k_cnt; v.q2k_idx = m->q2k_idx;
  v.k2q_cnt = m->k2q_cnt; v.k2q_idx = m->k2q_idx; v.status = m->status;
  v.q_order = m->q_order; v.k_order = m->k_order; v.totals = m->totals;
  return v;
}

}  // namespace

extern "C" {

const char* pba_strerror(int code) {
  switch (code) {
    case PBA_OK: return "ok";
    case PBA_ERR_NULL: return "a required pointer is NULL";
    case PBA_ERR_SHAPE: return "B, S, pack count or head count out of range";
    case PBA_ERR_HEADS: return "Hq is not a multiple of Hkv";
    case PBA_ERR_HEAD_DIM: return "head dim must be 64 or 128";
    case PBA_ERR_TILE: return "tile shape unsupported or map built for another tile shape";
    case PBA_ERR_MAP: return "map built for another (B, S) or its buffer is too small";
    case PBA_ERR_WORKSPACE: return "backward workspace missing or too small";
    case PBA_ERR_DEVICE: return "no gfx950 device current, or a HIP launch failed";
    case PBA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case PBA_ERR_SCALE: return "softmax scale must be positive and finite";
    case PBA_ERR_ARG: return "objective, beta, alpha or rotary base out of range";
    case PBA_ERR_SCRATCH: return "problem too large for the no-allocation backward's scratch (8*B*Hq*S bytes of row statistics must fit)";
    case PBA_DESC_ROW: return "descriptor: row outside [0, B)";
    case PBA_DESC_NEGATIVE: return "descriptor: negative start, length or response count";
    case PBA_DESC_RESP_RANGE: return "descriptor: response range outside resp_len";
    case PBA_DESC_BOUNDS: return "descriptor: pack runs past the end of its row";
    case PBA_DESC_ORDER: return "descriptor: packs not sorted by (row, start) or overlapping";
    case PBA_GROUP_BAD_PTR: return "groups: group_ptr not non-decreasing from 0 to n_entries";
    case PBA_GROUP_BAD_MEMBER: return "groups: member outside [0, n_resp)";
    case PBA_GROUP_BAD_LENGTH: return "groups: member response length not positive";
    case PBA_GROUP_DUPLICATE: return "groups: response named twice in one group";
    case PBA_GROUP_EMPTY_SET: return "groups: group without a positive or without a negative";
    default: return "unknown code";
  }
}

int pba_fwd_tile(int Hq, int Hkv, int D, int* block_m, int* block_n) {
  if (!block_m || !block_n) return PBA_ERR_NULL;
  if (Hq < 1 || Hkv < 1 || Hq > kMaxHeads) return PBA_ERR_SHAPE;
  if (Hq % Hkv) return PBA_ERR_HEADS;
  if (D != 64 && D != 128) return PBA_ERR_HEAD_DIM;
  *block_m = pba::kFwdBM * (4 / pba::fwd_wg_heads(Hq / Hkv));
  *block_n = pba::kFwdBN;
  return PBA_OK;
}

int pba_bwd_tile(int Hq, int Hkv, int D, int* block_m, int* block_n) {
  if (!block_m || !block_n) return PBA_ERR_NULL;
  if (Hq < 1 || Hkv < 1 || Hq > kMaxHeads) return PBA_ERR_SHAPE;
  if (Hq % Hkv) return PBA_ERR_HEADS;
  if (D != 64 && D != 128) return PBA_ERR_HEAD_DIM;
  *block_m = pba::kBwdBM;
  *block_n = pba::kBwdBN;
  return PBA_OK;
}

size_t pba_map_bytes(int B, int S, int block_m, int block_n) {
  if (B < 1 || B > kMaxB || S < 1 || S > kMaxS || !tile_ok(block_m) || !tile_ok(block_n)) return 0;
  return map_layout(B, S, block_m, block_n).total;
}

int pba_map_init(pba_block_map* map, void* buffer, size_t buffer_bytes, int B, int S, int block_m, int block_n) {
  if (!map || !buffer) return PBA_ERR_NULL;
  if (B < 1 || B > kMaxB || S < 1 || S > kMaxS) return PBA_ERR_SHAPE;
  if (!tile_ok(block_m) || !tile_ok(block_n)) return PBA_ERR_TILE;
  if ((reinterpret_cast<uintptr_t>(buffer) & (kAlign - 1)) != 0) return PBA_ERR_ALIGN;
  const MapLayout L = map_layout(B, S, block_m, block_n);
  if (buffer_bytes < L.total) return PBA_ERR_MAP;
  char* base = static_cast<char*>(buffer);
  map->B = B;
  map->S = S;
  map->block_m = block_m;
  map->block_n = block_n;
  map->nqt = (S + block_m - 1) / block_m;
  map->nkt = (S + block_n - 1) / block_n;
  map->tok_pack = reinterpret_cast<int32_t*>(base + L.off[0]);
  map->tok_branch = reinterpret_cast<int32_t*>(base + L.off[1]);
  map->tok_win = reinterpret_cast<int32_t*>(base + L.off[2]);
  map->cls = reinterpret_cast<uint8_t*>(base + L.off[3]);
  map->q2k_cnt = reinterpret_cast<int32_t*>(base + L.off[4]);
  map->q2k_idx = reinterpret_cast<int32_t*>(base + L.off[5]);
  map->k2q_cnt = reinterpret_cast<int32_t*>(base + L.off[6]);
  map->k2q_idx = reinterpret_cast<int32_t*>(base + L.off[7]);
  map->totals = reinterpret_cast<int64_t*>(base + L.off[8]);
  map->status = reinterpret_cast<int32_t*>(base + L.off[9]);
  map->q_order = reinterpret_cast<int32_t*>(base + L.off[10]);
  map->k_order = reinterpret_cast<int32_t*>(base + L.off[11]);
  map->work = reinterpret_cast<int32_t*>(base + L.off[12]);
  return PBA_OK;
}

int pba_pack_block_maps(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                        const pba_block_map* maps, int n_maps, void* stream) {
  if (!maps) return PBA_ERR_NULL;
  if (n_maps < 1 || n_maps > PBA_MAX_MAPS_PER_BUILD) return PBA_ERR_SHAPE;
  if (n_packs < 0 || n_resp_total < 0) return PBA_ERR_SHAPE;
  if ((n_packs > 0 && !packs) || (n_resp_total > 0 && !resp_len)) return PBA_ERR_NULL;
  for (int i = 0; i < n_maps; ++i) {
    const pba_block_map* map = maps + i;
    if (!map->tok_pack || !map->tok_branch || !map->tok_win || !map->cls || !map->q2k_cnt || !map->q2k_idx ||
        !map->k2q_cnt || !map->k2q_idx || !map->totals || !map->status || !map->q_order || !map->k_order ||
        !map->work)
      return PBA_ERR_NULL;
    if (map->B < 1 || map->B > kMaxB || map->S < 1 || map->S > kMaxS) return PBA_ERR_SHAPE;
    if (map->B != maps[0].B || map->S != maps[0].S) return PBA_ERR_MAP;
    if (!tile_ok(map->block_m) || !tile_ok(map->block_n)) return PBA_ERR_TILE;
    if (map->nqt != (map->S + map->block_m - 1) / map->block_m ||
        map->nkt != (map->S + map->block_n - 1) / map->block_n)
      return PBA_ERR_MAP;
  }
  if (int rc = device_ok()) return rc;
  hipError_t e = pba::launch_maps(packs, n_packs, resp_len, n_resp_total, maps, n_maps,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int pba_pack_positions(const pba_block_map* map, int32_t* pos_ids, int32_t* src_row, uint8_t* loss_mask,
                       void* stream) {
  if (!map || !map->tok_pack || !map->tok_branch || !map->tok_win || !map->status) return PBA_ERR_NULL;
  if (map->B < 1 || map->B > kMaxB || map->S < 1 || map->S > kMaxS) return PBA_ERR_SHAPE;
  if (!pos_ids && !src_row && !loss_mask) return PBA_OK;
  if (int rc = device_ok()) return rc;
  pba::PosArgs a;
  a.ntok = (int64_t)map->B * map->S;
  a.S = map->S;
  a.status = map->status;
  a.tok_pack = map->tok_pack;
  a.tok_branch = map->tok_branch;
  a.tok_win = map->tok_win;
  a.pos = pos_ids;
  a.src = src_row;
  a.mask = loss_mask;
  return pba::launch_positions(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int pba_packed_token_logp(const pba_block_map* map, const pba_pack* packs, int n_packs, const int32_t* resp_len,
                          int n_resp_total, const int32_t* src_row, const uint8_t* loss_mask, const void* logits,
                          int V, const int32_t* tokens, float* tok_logp, float* resp_logp, void* stream) {
  if (!map || !map->status || !src_row || !loss_mask || !logits || !tokens || !tok_logp) return PBA_ERR_NULL;
  if (map->B < 1 || map->B > kMaxB || map->S < 1 || map->S > kMaxS) return PBA_ERR_SHAPE;
  if (V < 8 || V % 8 != 0) return PBA_ERR_SHAPE;
  if (!aligned16(logits)) return PBA_ERR_ALIGN;
  if (resp_logp) {
    if (n_packs < 0 || n_resp_total < 0) return PBA_ERR_SHAPE;
    if ((n_packs > 0 && !packs) || (n_resp_total > 0 && !resp_len)) return PBA_ERR_NULL;
  }
  if (int rc = device_ok()) return rc;
  pba::LogpArgs a;
  a.status = map->status;
  a.logits = static_cast<const pba::bf16*>(logits);
  a.V = V;
  a.ntok = (int64_t)map->B * map->S;
  a.S = map->S;
  a.tokens = tokens;
  a.src = src_row;
  a.mask = loss_mask;
  a.tok_logp = tok_logp;
  pba::RespSumArgs r;
  r.status = map->status;
  r.packs = packs;
  r.n_packs = n_packs;
  r.S = map->S;
  r.resp_len = resp_len;
  r.tok_logp = tok_logp;
  r.resp_logp = resp_logp;
  return pba::launch_token_logp(a, resp_logp ? &r : nullptr, static_cast<hipStream_t>(stream)) == hipSuccess
             ? PBA_OK
             : PBA_ERR_DEVICE;
}

int pba_packed_rope(const pba_block_map* map, const void* x, void* y, int H, int D, float base, int inverse,
                    void* stream) {
  if (!map || !map->status || !map->tok_pack || !map->tok_win || !x || !y) return PBA_ERR_NULL;
  if (map->B < 1 || map->B > kMaxB || map->S < 1 || map->S > kMaxS || H < 1 || H > kMaxHeads) return PBA_ERR_SHAPE;
  if (D != 64 && D != 128) return PBA_ERR_HEAD_DIM;
  if (!(base > 1.f) || !std::isfinite(base)) return PBA_ERR_ARG;
  if (!aligned16(x) || !aligned16(y)) return PBA_ERR_ALIGN;
  if (int rc = device_ok()) return rc;
  pba::RopeArgs a;
  a.status = map->status;
  a.tok_pack = map->tok_pack;
  a.tok_win = map->tok_win;
  a.x = static_cast<const pba::bf16*>(x);
  a.y = static_cast<pba::bf16*>(y);
  a.ntok = (int64_t)map->B * map->S;
  a.S = map->S;
  a.H = H;
  a.log2_base = std::log2(base);
  a.sign = inverse ? -1.f : 1.f;
  return pba::launch_rope(a, D, static_cast<hipStream_t>(stream)) == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int pba_group_coefficients(const int32_t* group_ptr, int n_groups, const int32_t* member, const uint8_t* positive,
                           int n_entries, const float* pol, const float* ref, const int32_t* resp_len, int n_resp,
                           int objective, float beta, float alpha, float* coef, float* nll_w, float* loss,
                           int32_t* status, void* stream) {
  if (!group_ptr || !member || !positive || !pol || !ref || !resp_len || !coef || !status) return PBA_ERR_NULL;
  if (n_entries < 2 || n_entries > PBA_GROUP_MAX_ENTRIES || n_groups < 1 || n_groups > n_entries / 2 || n_resp < 1)
    return PBA_ERR_SHAPE;
  if (objective < PBA_GROUP_ALL_PAIRS || objective > PBA_GROUP_SOFTMAX) return PBA_ERR_ARG;
  if (!(beta > 0.f) || !std::isfinite(beta) || !(alpha >= 0.f) || !std::isfinite(alpha)) return PBA_ERR_ARG;
  if (int rc = device_ok()) return rc;
  pba::GroupArgs a;
  a.group_ptr = group_ptr;
  a.member = member;
  a.positive = positive;
  a.pol = pol;
  a.ref = ref;
  a.resp_len = resp_len;
  a.n_groups = n_groups;
  a.n_entries = n_entries;
  a.n_resp = n_resp;
  a.objective = objective;
  a.beta = beta;
  a.alpha = alpha;
  a.coef = coef;
  a.nll_w = nll_w;
  a.loss = loss;
  a.status = status;
  return pba::launch_group_coef(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int pba_pack_block_map(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                       const pba_block_map* map, void* stream) {
  return pba_pack_block_maps(packs, n_packs, resp_len, n_resp_total, map, 1, stream);
}

}  // extern "C"

namespace {
int fwd_impl(const pba_block_map* map, const void* q, const void* k, const void* v, void* o, float* lse, void* q_rot,
             int B, int S, int Hq, int Hkv, int D, float softmax_scale, float rope_base, void* stream) {
  if (!q || !k || !v || !o || !lse) return PBA_ERR_NULL;
  if (int rc = check_heads(B, S, Hq, Hkv, D)) return rc;
  if (int rc = check_scale(softmax_scale)) return rc;
  if (int rc = check_row_bytes(S, Hq, D)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (q_rot && !aligned16(q_rot)))
    return PBA_ERR_ALIGN;
  int bm, bn;
  pba_fwd_tile(Hq, Hkv, D, &bm, &bn);
  if (int rc = check_map(map, B, S, bm, bn)) return rc;
  if (int rc = device_ok()) return rc;
  pba::FwdArgs a;
  a.map = view_of(map);
  a.q = static_cast<const pba::bf16*>(q);
  a.k = static_cast<const pba::bf16*>(k);
  a.v = static_cast<const pba::bf16*>(v);
  a.o = static_cast<pba::bf16*>(o);
  a.lse = lse;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.wg_heads = pba::fwd_wg_heads(a.G);
  a.scale_log2 = softmax_scale * pba::kLog2eHost;
  a.rope_log2_base = rope_base > 0.f ? std::log2(rope_base) : 0.f;
  a.q_rot = static_cast<pba::bf16*>(q_rot);
  hipError_t e = pba::launch_fwd(a, D, B, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}
}  // namespace

extern "C" {

int pba_packed_attn_fwd(const pba_block_map* map, const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int S, int Hq, int Hkv, int D, float softmax_scale, void* stream) {
  return fwd_impl(map, q, k, v, o, lse, nullptr, B, S, Hq, Hkv, D, softmax_scale, 0.f, stream);
}

int pba_packed_attn_fwd_rope(const pba_block_map* map, const void* q, const void* k_rot, const void* v, void* o,
                             float* lse, void* q_rot, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                             float rope_base, void* stream) {
  if (!(rope_base > 1.f) || !std::isfinite(rope_base)) return PBA_ERR_ARG;
  return fwd_impl(map, q, k_rot, v, o, lse, q_rot, B, S, Hq, Hkv, D, softmax_scale, rope_base, stream);
}

size_t pba_bwd_workspace_bytes(int B, int S, int Hq, int D) {
  if (B < 1 || B > kMaxB || S < 1 || S > kMaxS || Hq < 1 || Hq > kMaxHeads || (D != 64 && D != 128)) return 0;
  return bwd_scratch_bytes(B, S, Hq, D, split_pairs(B, S, Hq));
}

}  // extern "C"

namespace {
// Bytes of the backward's scratch with `pairs` split pairs: -Delta and
// -LSE / scale (fp32 [B, Hq, S] each), pairs + 1 arrival counters, the partial sums.
size_t bwd_scratch_bytes(int B, int S, int Hq, int D, size_t pairs) {
  return 2 * align_up((size_t)B * Hq * S * 4) + align_up((pairs + 1) * 4) + pairs * 2 * 2 * pba::kBwdBN * D * 4;
}

// Host checks shared by every backward entry point.
int bwd_check(int stages, const pba_block_map* qmap, const pba_block_map* kmap, const void* q, const void* k,
              const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, int B,
              int S, int Hq, int Hkv, int D, float softmax_scale) {
  if (stages < 1 || stages > PBA_BWD_ALL) return PBA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return PBA_ERR_NULL;
  if (int rc = check_heads(B, S, Hq, Hkv, D)) return rc;
  if (int rc = check_scale(softmax_scale)) return rc;
  if (int rc = check_row_bytes(S, Hq, D)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return PBA_ERR_ALIGN;
  int bm, bn;
  pba_fwd_tile(Hq, Hkv, D, &bm, &bn);
  if (int rc = check_map(qmap, B, S, bm, bn)) return rc;
  pba_bwd_tile(Hq, Hkv, D, &bm, &bn);
  if (int rc = check_map(kmap, B, S, bm, bn)) return rc;
  return PBA_OK;
}

// Enqueues the backward's kernels with their scratch at `ws` (256-byte
// aligned, bwd_scratch_bytes(..., pairs) bytes) after bwd_check passed.
int bwd_launch(int stages, const pba_block_map* qmap, const pba_block_map* kmap, const void* q, const void* k,
               const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
               void* ws, size_t pairs, int B, int S, int Hq, int Hkv, int D, float softmax_scale, float rope_base,
               void* stream) {
  pba::BwdArgs a;
  a.qmap = view_of(qmap);
  a.kmap = view_of(kmap);
  a.q = static_cast<const pba::bf16*>(q);
  a.k = static_cast<const pba::bf16*>(k);
  a.v = static_cast<const pba::bf16*>(v);
  a.o = static_cast<const pba::bf16*>(o);
  a.lse = lse;
  a.dout = static_cast<const pba::bf16*>(dout);
  a.dq = static_cast<pba::bf16*>(dq);
  a.dk = static_cast<pba::bf16*>(dk);
  a.dv = static_cast<pba::bf16*>(dv);
  a.dp0 = static_cast<float*>(ws);
  a.s0 = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)B * Hq * S * 4));
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * pba::kLog2eHost;
  a.rope_log2_base = rope_base > 0.f ? std::log2(rope_base) : 0.f;
  // Split area: arrival counters, then the partial sums.
  char* split_base = static_cast<char*>(ws) + 2 * align_up((size_t)B * Hq * S * 4);
  a.arrive = reinterpret_cast<int32_t*>(split_base);
  a.part = reinterpret_cast<float*>(split_base + align_up((pairs + 1) * 4));
  const int fixed_slots = g_split_slots.load(std::memory_order_relaxed);
  a.slots = fixed_slots > 0 ? fixed_slots : std::max(1, cu_count() / Hkv);
  a.nsplit = (int)std::min({(size_t)B * kmap->nkt, (size_t)a.slots, pairs / (size_t)Hkv});
  hipError_t e = pba::launch_bwd(a, D, stages, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int bwd_impl(int stages, const pba_block_map* qmap, const pba_block_map* kmap, const void* q, const void* k,
             const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
             float rope_base, void* stream) {
  if (int rc = bwd_check(stages, qmap, kmap, q, k, v, o, lse, dout, dq, dk, dv, B, S, Hq, Hkv, D, softmax_scale))
    return rc;
  const size_t pairs = split_pairs(B, S, Hq);
  if (!workspace || workspace_bytes < bwd_scratch_bytes(B, S, Hq, D, pairs)) return PBA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return PBA_ERR_ALIGN;
  if (int rc = device_ok()) return rc;
  return bwd_launch(stages, qmap, kmap, q, k, v, o, lse, dout, dq, dk, dv, workspace, pairs, B, S, Hq, Hkv, D,
                    softmax_scale, rope_base, stream);
}
}  // namespace

namespace {
// Scratch of pba_packed_attn_bwd_noalloc: file-scope device memory, one copy
// per device, held until the process ends.  On the host, `scratch` names
// only a stand-in, not device memory: host code uses the device address
// that hipGetSymbolAddress returns, taken once per device and kept.
__device__ __align__(256) unsigned char scratch[PBA_NOALLOC_SCRATCH_BYTES];

// Device address of this device's `scratch` (nullptr if it cannot be had).
void* scratch_address() {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

// Split pairs that fit the scratch next to the per-row arrays (at most the
// workspace's own count, so results match pba_packed_attn_bwd whenever they
// all fit); -1 when those arrays and one counter alone do not fit.
long long noalloc_pairs(int B, int S, int Hq, int D) {
  size_t pairs = split_pairs(B, S, Hq);
  if (bwd_scratch_bytes(B, S, Hq, D, 0) > PBA_NOALLOC_SCRATCH_BYTES) return -1;
  while (pairs > 0 && bwd_scratch_bytes(B, S, Hq, D, pairs) > PBA_NOALLOC_SCRATCH_BYTES) --pairs;
  return (long long)pairs;
}
}  // namespace

extern "C" {

int pba_packed_attn_bwd_stages(int stages, const pba_block_map* qmap, const pba_block_map* kmap, const void* q,
                               const void* k, const void* v, const void* o, const float* lse, const void* dout,
                               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int S,
                               int Hq, int Hkv, int D, float softmax_scale, void* stream) {
  return bwd_impl(stages, qmap, kmap, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, S, Hq, Hkv, D,
                  softmax_scale, 0.f, stream);
}

int pba_packed_attn_bwd_rope(const pba_block_map* qmap, const pba_block_map* kmap, const void* q_rot,
                             const void* k_rot, const void* v, const void* o, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int S,
                             int Hq, int Hkv, int D, float softmax_scale, float rope_base, void* stream) {
  if (!(rope_base > 1.f) || !std::isfinite(rope_base)) return PBA_ERR_ARG;
  return bwd_impl(PBA_BWD_ALL, qmap, kmap, q_rot, k_rot, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B,
                  S, Hq, Hkv, D, softmax_scale, rope_base, stream);
}

int pba_packed_attn_bwd_noalloc(const pba_block_map* qmap, const pba_block_map* kmap, const void* q,
                                const void* k, const void* v, const void* o, const float* lse, const void* dout,
                                void* dq, void* dk, void* dv, int B, int S, int Hq, int Hkv, int D,
                                float softmax_scale, void* stream) {
  if (int rc = bwd_check(PBA_BWD_ALL, qmap, kmap, q, k, v, o, lse, dout, dq, dk, dv, B, S, Hq, Hkv, D,
                         softmax_scale))
    return rc;
  const long long pairs = noalloc_pairs(B, S, Hq, D);
  if (pairs < 0) return PBA_ERR_SCRATCH;
  if (int rc = device_ok()) return rc;
  void* ws = scratch_address();
  if (!ws) return PBA_ERR_DEVICE;
  return bwd_launch(PBA_BWD_ALL, qmap, kmap, q, k, v, o, lse, dout, dq, dk, dv, ws, (size_t)pairs, B, S, Hq, Hkv, D,
                    softmax_scale, 0.f, stream);
}

int pba_set_bwd_split_slots(int slots) {
  if (slots < 0) return PBA_ERR_SHAPE;
  return g_split_slots.exchange(slots);
}

int pba_packed_attn_bwd(const pba_block_map* qmap, const pba_block_map* kmap, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int S, int Hq, int Hkv, int D,
                        float softmax_scale, void* stream) {
  return pba_packed_attn_bwd_stages(PBA_BWD_ALL, qmap, kmap, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                    workspace_bytes, B, S, Hq, Hkv, D, softmax_scale, stream);
}

}  // extern "C"

namespace pba {
hipError_t launch_mfma_probe(float* out, int n_blocks, int iters, hipStream_t stream);  // pba_probe.hip
hipError_t launch_lds_probe(float* out, int n_blocks, int iters, hipStream_t stream);
hipError_t launch_valu_probe(float* out, int n_blocks, int iters, int exp, hipStream_t stream);
}

extern "C" {

int pba_mfma_probe(float* out, int n_blocks, int iters, void* stream) {
  if (!out) return PBA_ERR_NULL;
  if (n_blocks < 1 || n_blocks > (1 << 20) || iters < 1) return PBA_ERR_SHAPE;
  if (int rc = device_ok()) return rc;
  return pba::launch_mfma_probe(out, n_blocks, iters, (hipStream_t)stream) == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int pba_lds_probe(float* out, int n_blocks, int iters, void* stream) {
  if (!out) return PBA_ERR_NULL;
  if (n_blocks < 1 || n_blocks > (1 << 20) || iters < 1) return PBA_ERR_SHAPE;
  if (int rc = device_ok()) return rc;
  return pba::launch_lds_probe(out, n_blocks, iters, (hipStream_t)stream) == hipSuccess ? PBA_OK : PBA_ERR_DEVICE;
}

int pba_valu_probe(float* out, int n_blocks, int iters, int exp2, void* stream) {
  if (!out) return PBA_ERR_NULL;
  if (n_blocks < 1 || n_blocks > (1 << 20) || iters < 1 || (exp2 != 0 && exp2 != 1)) return PBA_ERR_SHAPE;
  if (int rc = device_ok()) return rc;
  return pba::launch_valu_probe(out, n_blocks, iters, exp2, (hipStream_t)stream) == hipSuccess ? PBA_OK
                                                                                             : PBA_ERR_DEVICE;
}

}  // extern "C"
