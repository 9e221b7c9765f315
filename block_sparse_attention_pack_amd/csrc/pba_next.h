// Declarations shared by the kernels of the rows that follow attention
// (positions and log-prob gathering) and the C-ABI layer.
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

}  // namespace pba
