// Internal declarations shared by the library's translation units (not part
// of the C ABI).  gfx950 only: wave64, bf16 MFMA, LDS transpose reads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pba.h"

namespace pba {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define PBA_LDS __attribute__((address_space(3)))

// Tile shapes of the attention kernels (query tokens x key tokens).
constexpr int kFwdBM = 32;   // one wave owns 32 query rows of one q head
constexpr int kFwdBN = 64;
constexpr int kBwdBM = 64;   // query rows per dK / dV step
constexpr int kBwdBN = 128;  // key rows per dK / dV workgroup (4 waves x 32)

struct MapView {  // device-side view of a pba_block_map
  int B, S, bm, bn, nqt, nkt;
  const int32_t* tok_win;
  const int32_t* q2k_cnt;
  const int32_t* q2k_idx;
  const int32_t* k2q_cnt;
  const int32_t* k2q_idx;
  const int32_t* status;
  const int32_t* q_order;  // [B*nqt] query tiles, longest visit list first
  const int32_t* k_order;  // [B*nkt] key tiles, longest visit list first
  const int64_t* totals;   // [3] full, partial, skipped tiles
};

struct FwdArgs {
  MapView map;
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int S, Hq, Hkv, G, wg_heads;
  float scale_log2;  // softmax scale * log2(e)
  // Rotary inputs: Q is rotated at the packed positions inside the kernel
  // (log2 of the base; 0 = Q is used as given) and, if q_rot is not null,
  // written there for the backward.
  float rope_log2_base;
  bf16* q_rot;
};

struct BwdArgs {
  MapView qmap;  // query-major map, forward tile shape (bwd_dq)
  MapView kmap;  // key-major map, backward tile shape (bwd_dkdv)
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  // Written by bwd_dq for bwd_dkdv: the values its dP and score
  // accumulators start from, so that the finished accumulators are dP - Delta
  // and S - LSE / scale (whose exp2(scale * log2(e) * x) is P).
  float* dp0;  // [B, Hq, S] fp32 -Delta = -rowsum(dO * O)
  float* s0;   // [B, Hq, S] fp32 -LSE / scale (0 for rows that see nothing)
  int B, S, Hq, Hkv, G;
  float scale, scale_log2;
  // log2 of the rotary base when dQ and dK are rotated back to the
  // unrotated Q and K (the inputs were rotated at the packed positions);
  // 0 = no rotation.
  float rope_log2_base;
  // Key tiles whose visit list is longer than the average load of one
  // workgroup slot are split between two workgroups (bwd_dkdv): the first
  // nsplit work-order positions may be split; their halves' fp32 partial
  // sums meet in `part` ([nsplit*Hkv][2 halves][2 tensors][4 key blocks]
  // [D/8][64 lanes] x 4 floats), counted in `arrive` ([nsplit*Hkv], zeroed
  // by bwd_dq, followed by the number of positions actually split, also
  // written by bwd_dq).  slots = workgroup slots per kv group (CUs / Hkv,
  // >= 1).
  float* part;
  int32_t* arrive;
  int nsplit, slots;
};

// Upper bound on nsplit * Hkv (sizes the split area of the workspace).
constexpr int kMaxSplitPairs = 256;

constexpr float kLog2eHost = 1.4426950408889634f;

// Launchers (return hipError_t of the launch).
constexpr int kMaxMapsPerBuild = PBA_MAX_MAPS_PER_BUILD;
hipError_t launch_maps(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                       const pba_block_map* maps, int n_maps, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int D, int B, hipStream_t stream);
// Backward stages (bit mask): dQ (and Delta, LSE2), then dK / dV.
constexpr int kBwdDq = 1, kBwdDkdv = 2, kBwdAll = 3;
hipError_t launch_bwd(const BwdArgs& a, int D, int stages, hipStream_t stream);
// q heads per forward / dQ workgroup for G q heads per kv head.
int fwd_wg_heads(int G);

}  // namespace pba
