// Declarations shared by the kernels of the rows that follow attention
// (positions, rotary embedding, log-prob gathering, group preference
// coefficients) and the C-ABI layer.
#pragma once

#include "pba_internal.h"

namespace pba {

struct PosArgs {  // map_positions
  int64_t ntok;
  int S;
  const int32_t* status;
  const int32_t* tok_pack;
  const int32_t* tok_branch;
  const int32_t* tok_win;
  int32_t* pos;
  int32_t* src;
  uint8_t* mask;
};
hipError_t launch_positions(const PosArgs& a, hipStream_t stream);

struct LogpArgs {  // token_logp
  const int32_t* status;
  const bf16* logits;
  int64_t V, ntok;
  int S;
  const int32_t* tokens;
  const int32_t* src;
  const uint8_t* mask;
  float* tok_logp;
};
struct RespSumArgs {  // resp_logp
  const int32_t* status;
  const pba_pack* packs;
  int n_packs, S;
  const int32_t* resp_len;
  const float* tok_logp;
  float* resp_logp;
};
hipError_t launch_token_logp(const LogpArgs& a, const RespSumArgs* r, hipStream_t stream);

constexpr int kMaxGroupEntries = PBA_GROUP_MAX_ENTRIES;
constexpr int kMaxGroups = PBA_GROUP_MAX_ENTRIES / 2;  // every group has at least two entries
enum : int {
  kObjAllPairs = PBA_GROUP_ALL_PAIRS,
  kObjMargin = PBA_GROUP_MARGIN,
  kObjMpo = PBA_GROUP_MPO,
  kObjSoftmax = PBA_GROUP_SOFTMAX,
  kGroupPtr = PBA_GROUP_BAD_PTR,
  kGroupMember = PBA_GROUP_BAD_MEMBER,
  kGroupLength = PBA_GROUP_BAD_LENGTH,
  kGroupDuplicate = PBA_GROUP_DUPLICATE,
  kGroupEmpty = PBA_GROUP_EMPTY_SET,
};
struct GroupArgs {  // group_coef
  const int32_t* group_ptr;
  const int32_t* member;
  const uint8_t* positive;
  const float* pol;
  const float* ref;
  const int32_t* resp_len;
  int n_groups, n_entries, n_resp, objective;
  double beta, alpha;
  float* coef;
  float* nll_w;
  float* loss;
  int32_t* status;
};
hipError_t launch_group_coef(const GroupArgs& a, hipStream_t stream);

struct RopeArgs {  // rope_apply
  const int32_t* status;
  const int32_t* tok_pack;
  const int32_t* tok_win;
  const bf16* x;
  bf16* y;
  int64_t ntok;
  int S, H;
  float log2_base, sign;
};
hipError_t launch_rope(const RopeArgs& a, int D, hipStream_t stream);

}  // namespace pba
