// Host-side argument checks of the C ABI under AddressSanitizer.
//
// Built by tests/test_asan_host.py with the host half of pba_api.cpp
// instrumented (hipcc -Xarch_host -fsanitize=address) and linked with the
// library's other objects; run on a machine without a GPU.  Every call below
// is rejected by the host layer before any device work (null pointers, shapes,
// map mismatches, scale, workspace, alignment, the no-allocation backward's
// scratch limit), so ASan sees every byte the checks and the map carving
// touch.  Exit status 0 iff every call returns the expected code.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../include/pba.h"
#include "../include/pba_measure.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                         \
  do {                                                                             \
    const int got_ = (call);                                                       \
    if (got_ != (want)) {                                                          \
      std::printf("FAIL line %d: %s = %d, expected %d\n", __LINE__, #call, got_, want); \
      ++g_fail;                                                                    \
    }                                                                              \
  } while (0)

int main() {
  // A fake device address: the host layer only checks and carves it.
  void* const buf = reinterpret_cast<void*>(uintptr_t(1) << 20);
  void* const p16 = reinterpret_cast<void*>(uintptr_t(16));
  int bm = 0, bn = 0;
  EXPECT(pba_fwd_tile(32, 8, 128, &bm, &bn), PBA_OK);
  if (bm != 32 || bn != 64) ++g_fail;
  EXPECT(pba_fwd_tile(32, 7, 128, &bm, &bn), PBA_ERR_HEADS);
  EXPECT(pba_fwd_tile(32, 8, 96, &bm, &bn), PBA_ERR_HEAD_DIM);
  EXPECT(pba_fwd_tile(32, 8, 128, nullptr, &bn), PBA_ERR_NULL);
  EXPECT(pba_bwd_tile(0, 8, 128, &bm, &bn), PBA_ERR_SHAPE);
  if (pba_map_bytes(0, 10, 64, 64) != 0 || pba_map_bytes(1, 10, 48, 64) != 0) ++g_fail;
  if (pba_bwd_workspace_bytes(1, 10, 4, 80) != 0) ++g_fail;

  pba_block_map m, mb, big_q, big_k;
  std::memset(&m, 0, sizeof m);
  EXPECT(pba_map_init(&m, buf, 1 << 20, 2, 100, 64, 64), PBA_OK);
  EXPECT(pba_map_init(&mb, buf, 1 << 20, 2, 100, 64, 128), PBA_OK);
  EXPECT(pba_map_init(&m, reinterpret_cast<char*>(buf) + 16, 1 << 20, 2, 100, 64, 64), PBA_ERR_ALIGN);
  EXPECT(pba_map_init(&m, buf, 16, 2, 100, 64, 64), PBA_ERR_MAP);
  EXPECT(pba_map_init(&m, buf, 1 << 20, 2, 100, 64, 64), PBA_OK);
  EXPECT(pba_map_init(nullptr, buf, 1 << 20, 2, 100, 64, 64), PBA_ERR_NULL);

  EXPECT(pba_pack_block_map(nullptr, 0, nullptr, 0, nullptr, nullptr), PBA_ERR_NULL);
  EXPECT(pba_pack_block_map(nullptr, 3, nullptr, 0, &m, nullptr), PBA_ERR_NULL);
  EXPECT(pba_pack_block_maps(nullptr, 0, nullptr, 0, &m, 0, nullptr), PBA_ERR_SHAPE);
  EXPECT(pba_pack_block_maps(nullptr, 0, nullptr, 0, &m, PBA_MAX_MAPS_PER_BUILD + 1, nullptr), PBA_ERR_SHAPE);

  // forward: null, map shape, tile, heads, alignment, scale, row size
  EXPECT(pba_packed_attn_fwd(nullptr, p16, p16, p16, p16, nullptr, 1, 8, 2, 2, 64, 0.1f, nullptr), PBA_ERR_NULL);
  EXPECT(pba_packed_attn_fwd(&m, p16, p16, p16, p16, (float*)p16, 2, 101, 4, 2, 64, 0.1f, nullptr), PBA_ERR_MAP);
  EXPECT(pba_packed_attn_fwd(&m, p16, p16, p16, p16, (float*)p16, 2, 100, 4, 4, 64, 0.1f, nullptr), PBA_ERR_TILE);
  EXPECT(pba_packed_attn_fwd(&m, p16, p16, p16, p16, (float*)p16, 2, 100, 4, 3, 64, 0.1f, nullptr), PBA_ERR_HEADS);
  EXPECT(pba_packed_attn_fwd(&m, (void*)8, p16, p16, p16, (float*)p16, 2, 100, 4, 2, 64, 0.1f, nullptr),
         PBA_ERR_ALIGN);
  EXPECT(pba_packed_attn_fwd(&m, p16, p16, p16, p16, (float*)p16, 2, 100, 4, 2, 64, 0.0f, nullptr), PBA_ERR_SCALE);
  EXPECT(pba_packed_attn_fwd(&m, p16, p16, p16, p16, (float*)p16, 2, 100, 4, 2, 64, NAN, nullptr), PBA_ERR_SCALE);
  EXPECT(pba_packed_attn_fwd(&m, p16, p16, p16, p16, (float*)p16, 2, 1 << 20, 16, 8, 128, 0.1f, nullptr),
         PBA_ERR_SHAPE);
  EXPECT(pba_packed_attn_fwd_rope(&m, p16, p16, p16, p16, (float*)p16, nullptr, 2, 100, 4, 2, 64, 0.1f, 1.0f,
                                  nullptr),
         PBA_ERR_ARG);

  // backward: workspace size and alignment, swapped maps, scale, stage mask
  const size_t ws = pba_bwd_workspace_bytes(2, 100, 4, 64);
  EXPECT(pba_packed_attn_bwd(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, buf, 0, 2, 100, 4, 2, 64,
                             0.1f, nullptr),
         PBA_ERR_WORKSPACE);
  EXPECT(pba_packed_attn_bwd(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, buf, ws - 1, 2, 100, 4, 2,
                             64, 0.1f, nullptr),
         PBA_ERR_WORKSPACE);
  EXPECT(pba_packed_attn_bwd(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16,
                             reinterpret_cast<char*>(buf) + 64, ws, 2, 100, 4, 2, 64, 0.1f, nullptr),
         PBA_ERR_ALIGN);
  EXPECT(pba_packed_attn_bwd(&mb, &m, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, buf, ws, 2, 100, 4, 2, 64,
                             0.1f, nullptr),
         PBA_ERR_TILE);
  EXPECT(pba_packed_attn_bwd(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, buf, ws, 2, 100, 4, 2, 64,
                             INFINITY, nullptr),
         PBA_ERR_SCALE);
  EXPECT(pba_packed_attn_bwd_stages(0, &m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, buf, ws, 2, 100,
                                    4, 2, 64, 0.1f, nullptr),
         PBA_ERR_SHAPE);
  EXPECT(pba_packed_attn_bwd_rope(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, buf, ws, 2, 100, 4, 2,
                                  64, 0.1f, -3.0f, nullptr),
         PBA_ERR_ARG);

  // no-allocation backward: checks, then the scratch limit
  EXPECT(pba_packed_attn_bwd_noalloc(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, nullptr, 2, 100, 4, 2,
                                     64, 0.1f, nullptr),
         PBA_ERR_NULL);
  EXPECT(pba_packed_attn_bwd_noalloc(&m, &mb, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, 2, 100, 4, 2, 96,
                                     0.1f, nullptr),
         PBA_ERR_HEAD_DIM);
  EXPECT(pba_fwd_tile(32, 8, 128, &bm, &bn), PBA_OK);
  EXPECT(pba_map_init(&big_q, buf, size_t(1) << 40, 16, 32768, bm, bn), PBA_OK);
  EXPECT(pba_bwd_tile(32, 8, 128, &bm, &bn), PBA_OK);
  EXPECT(pba_map_init(&big_k, buf, size_t(1) << 40, 16, 32768, bm, bn), PBA_OK);
  EXPECT(pba_packed_attn_bwd_noalloc(&big_q, &big_k, p16, p16, p16, p16, (float*)p16, p16, p16, p16, p16, 16, 32768,
                                     32, 8, 128, 0.1f, nullptr),
         PBA_ERR_SCRATCH);

  // next rows
  EXPECT(pba_pack_positions(nullptr, (int32_t*)p16, nullptr, nullptr, nullptr), PBA_ERR_NULL);
  EXPECT(pba_pack_positions(&m, nullptr, nullptr, nullptr, nullptr), PBA_OK);
  EXPECT(pba_packed_token_logp(&m, nullptr, 0, nullptr, 0, (int32_t*)p16, (uint8_t*)p16, p16, 12, (int32_t*)p16,
                               (float*)p16, nullptr, nullptr),
         PBA_ERR_SHAPE);
  EXPECT(pba_packed_token_logp(&m, nullptr, 0, nullptr, 0, (int32_t*)p16, (uint8_t*)p16, (void*)8, 16, (int32_t*)p16,
                               (float*)p16, nullptr, nullptr),
         PBA_ERR_ALIGN);
  EXPECT(pba_packed_rope(&m, p16, p16, 4, 64, 0.5f, 0, nullptr), PBA_ERR_ARG);
  EXPECT(pba_packed_rope(&m, p16, p16, 4, 80, 1e4f, 0, nullptr), PBA_ERR_HEAD_DIM);
  EXPECT(pba_group_coefficients((int32_t*)p16, 1, (int32_t*)p16, (uint8_t*)p16, 1, (float*)p16, (float*)p16,
                                (int32_t*)p16, 1, 0, 0.1f, 1.0f, (float*)p16, nullptr, nullptr, (int32_t*)p16, nullptr),
         PBA_ERR_SHAPE);
  EXPECT(pba_group_coefficients((int32_t*)p16, 1, (int32_t*)p16, (uint8_t*)p16, 2, (float*)p16, (float*)p16,
                                (int32_t*)p16, 1, 7, 0.1f, 1.0f, (float*)p16, nullptr, nullptr, (int32_t*)p16, nullptr),
         PBA_ERR_ARG);
  EXPECT(pba_mfma_probe(nullptr, 1, 1, nullptr), PBA_ERR_NULL);
  EXPECT(pba_valu_probe((float*)p16, 1, 1, 2, nullptr), PBA_ERR_SHAPE);
  EXPECT(pba_set_bwd_split_slots(-1), PBA_ERR_SHAPE);
  EXPECT(pba_set_bwd_split_slots(5), 0);
  EXPECT(pba_set_bwd_split_slots(0), 5);

  for (int c = -12; c <= 15; ++c)
    if (!pba_strerror(c) || std::strlen(pba_strerror(c)) == 0) ++g_fail;
  std::printf("%s: %d failed checks\n", g_fail ? "FAIL" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
