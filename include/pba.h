/*
 * pba.h -- packed branch-aware attention on MI355X (gfx950): C ABI.
 *
 * The operation.  A row of S tokens holds one or more packs laid out as
 * [prompt | response_0 | response_1 | ...] (the shared-prompt layout of
 * "DPO Preference Packing: Dense Masks and Sparse Execution", section
 * "Layout requirements"; K >= 2 responses after one prompt as in
 * "Preference Packing", section 3.1).  Query i may attend key j when both
 * lie in the same pack, j <= i, and j is a prompt token or lies in i's own
 * response: each response sees the shared prompt and its own earlier
 * tokens, never a sibling (same section), and nothing crosses a pack
 * boundary, as with cumulative-sequence-length packing ("Why does packing
 * several SFT examples into one sequence risk cross-example contamination?",
 * "The correct implementation"; "Pack training sequences to reduce padding
 * waste", the rule "same example AND key position <= query position").
 * Attention itself is ordinary masked softmax attention; tiles of the
 * score matrix that the mask empties are skipped, not computed
 * ("DPO Preference Packing", section "Dense and sparse execution").
 *
 * Three calls:
 *   pba_pack_block_map   descriptors -> per-token ids and windows, per-tile
 *                        class (skip / partial / full) and visit lists
 *   pba_packed_attn_fwd  Q, K, V (bf16, grouped heads) -> O (bf16), LSE (fp32)
 *   pba_packed_attn_bwd  dO -> dQ, dK, dV (bf16)
 * and the steps around them in a preference-training step: aligned
 * position ids and log-prob gather rows (pba_pack_positions), rotary
 * embedding at those positions (pba_packed_rope), packed token log-probs
 * (pba_packed_token_logp) and group preference coefficients
 * (pba_group_coefficients).
 *
 * Conventions shared by every call.
 *   - Every array argument is DEVICE memory allocated by the caller.  The
 *     library never allocates, never synchronises, never keeps a pointer
 *     after returning, and enqueues all work on `stream` (a hipStream_t;
 *     NULL = the default stream).
 *   - Host-visible argument errors return a negative PBA_ERR_* code and
 *     enqueue nothing.  Errors in descriptor CONTENTS can only be seen on the
 *     device: the map kernels record them in map->status (codes
 *     PBA_DESC_*), and then the map kernels and any later fwd/bwd call that
 *     uses that map write nothing.  Read map->status after a stream sync
 *     to check.
 *   - Layouts (row-major, contiguous): Q, O, dO, dQ [B, S, Hq, D];
 *     K, V, dK, dV [B, S, Hkv, D]; LSE [B, Hq, S].  q head h uses kv head
 *     h / (Hq / Hkv).  Pointers must be 16-byte aligned.
 *   - Output arrays (and a workspace) must not overlap any input array of
 *     the same call or each other: the kernels read inputs while other
 *     workgroups write outputs, so an overlap gives undefined values (it
 *     cannot make an access leave the arrays).  The library does not check
 *     this; the Python binding does.
 *   - Supported: D in {64, 128}; Hq % Hkv == 0; bf16 tensors; gfx950.
 *   - Pad tokens (inside a row but in no pack) must hold finite values; they
 *     never influence valid outputs and get O = 0, LSE = -inf and zero
 *     gradients.
 */
#ifndef PBA_H
#define PBA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PBA_API __attribute__((visibility("default")))
#else
#define PBA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes (host) ---------------------------------------------- */
#define PBA_OK              0
#define PBA_ERR_NULL       -1  /* a required pointer is NULL                      */
#define PBA_ERR_SHAPE      -2  /* B, S, n_packs, n_resp_total or a head count out of range */
#define PBA_ERR_HEADS      -3  /* Hq is not a multiple of Hkv                      */
#define PBA_ERR_HEAD_DIM   -4  /* D not in {64, 128}                               */
#define PBA_ERR_TILE       -5  /* tile shape unsupported, or map built for another tile shape */
#define PBA_ERR_MAP        -6  /* map built for another (B, S), or its buffer too small */
#define PBA_ERR_WORKSPACE  -7  /* backward workspace missing or too small           */
#define PBA_ERR_DEVICE     -8  /* no gfx950 device current, or a HIP launch failed  */
#define PBA_ERR_ALIGN      -9  /* a tensor pointer is not 16-byte aligned          */
#define PBA_ERR_SCALE     -10  /* softmax_scale not positive and finite            */
#define PBA_ERR_ARG       -11  /* objective, beta, alpha or rotary base out of range */
#define PBA_ERR_SCRATCH   -12  /* problem larger than the no-allocation backward's scratch */

/* ---- device status codes (map->status[0]; status[1] = first bad pack) -- */
#define PBA_DESC_OK          0
#define PBA_DESC_ROW         1  /* row outside [0, B)                                 */
#define PBA_DESC_NEGATIVE    2  /* negative start, prompt_len, n_resp or response length */
#define PBA_DESC_RESP_RANGE  3  /* resp_first / n_resp outside resp_len[]              */
#define PBA_DESC_BOUNDS      4  /* pack runs past the end of its row                   */
#define PBA_DESC_ORDER       5  /* packs not sorted by (row, start), or overlapping    */

/* ---- group status codes (pba_group_coefficients; status[1] = first bad group) */
#define PBA_GROUP_BAD_PTR     11  /* group_ptr not non-decreasing from 0 to n_entries   */
#define PBA_GROUP_BAD_MEMBER  12  /* member outside [0, n_resp)                         */
#define PBA_GROUP_BAD_LENGTH  13  /* member's response length not positive              */
#define PBA_GROUP_DUPLICATE   14  /* response twice in one group (or both signs)        */
#define PBA_GROUP_EMPTY_SET   15  /* group without a positive or without a negative     */

/* ---- tile classes in map->cls ------------------------------------------ */
#define PBA_TILE_SKIP     0
#define PBA_TILE_PARTIAL  1
#define PBA_TILE_FULL     2

/* One pack: tokens [start, start + prompt_len + sum of its response lengths)
 * of row `row`, prompt first, then responses resp_len[resp_first ..
 * resp_first + n_resp - 1] in order.  The descriptor array is sorted by
 * (row, start) with no overlaps; gaps between packs are pad.  A
 * cumulative-sequence-length batch maps to row = 0, start = cu[p] and one
 * response (or a prompt only) per pack.  Zero lengths are allowed. */
typedef struct {
  int32_t row;
  int32_t start;
  int32_t prompt_len;
  int32_t n_resp;
  int32_t resp_first;
} pba_pack;

/* The block map: a struct of device pointers into one caller-allocated
 * buffer, filled in by pba_map_init and written by pba_pack_block_map.
 * Tiles are block_m query tokens by block_n key tokens; nqt = ceil(S /
 * block_m), nkt = ceil(S / block_n); tokens at or beyond S count as pad, so
 * a tile touching them is never full.
 *   tok_pack[b*S+s]    pack index covering token s of row b, -1 for pad
 *   tok_branch[b*S+s]  0 in the prompt, k + 1 in response k, 0 for pad
 *   tok_win[(b*S+s)*4 + {0,1,2,3}] = {kv_lo, pre_lo, pre_hi, q_end}:
 *       as a query, token s sees keys [pre_lo, pre_hi) U [kv_lo, s]
 *       (pre_lo = pre_hi = 0 when its visible keys form one run; kv_lo = s+1
 *       for pad); as a key, it is seen by queries [s, q_end) (q_end = s for
 *       pad).  Indices are positions within the row.
 *   cls[(b*nqt+qt)*nkt+kt]     PBA_TILE_*
 *   q2k_cnt[(b*nqt+qt)*2+{0,1}] = {n_full, n_partial} of query tile qt;
 *   q2k_idx[(b*nqt+qt)*nkt + i] = its key tiles: full ones ascending, then
 *       partial ones ascending, then -1.
 *   k2q_cnt / k2q_idx: the same per key tile over query tiles ([B*nkt*2],
 *       [B*nkt*nqt]).
 *   totals[3] = {n_full, n_partial, n_skip} over all rows.
 *   status[2] = {PBA_DESC_* code, first offending pack or -1}.
 *   q_order[B*nqt]: the query tiles b*nqt + qt sorted by visit count
 *       (n_full + n_partial) descending, ties by index ascending: the
 *       order in which the query-major kernels take their work, longest
 *       first.  k_order[B*nkt]: the same for the key tiles.
 *   work: the map kernels' own scratch (histograms), contents unspecified. */
typedef struct {
  int32_t B, S, block_m, block_n, nqt, nkt;
  int32_t* tok_pack;
  int32_t* tok_branch;
  int32_t* tok_win;
  uint8_t* cls;
  int32_t* q2k_cnt;
  int32_t* q2k_idx;
  int32_t* k2q_cnt;
  int32_t* k2q_idx;
  int64_t* totals;
  int32_t* status;
  int32_t* q_order;
  int32_t* k_order;
  int32_t* work;
} pba_block_map;

/* Error message for a return code or device status code (static string). */
PBA_API const char* pba_strerror(int code);

/* Tile shape (query tokens x key tokens) the forward / backward kernels need
 * their map built with, for head dim D and the given head counts.  Returns
 * PBA_OK or an argument error; *block_m / *block_n receive the shape. */
PBA_API int pba_fwd_tile(int Hq, int Hkv, int D, int* block_m, int* block_n);
PBA_API int pba_bwd_tile(int Hq, int Hkv, int D, int* block_m, int* block_n);

/* Bytes of the single device buffer a map of this shape needs (0 on bad
 * arguments).  Supported tiles: block_m, block_n in {16, 32, 64, 128, 256}. */
PBA_API size_t pba_map_bytes(int B, int S, int block_m, int block_n);

/* Point `map` into `buffer` (device memory, >= pba_map_bytes bytes, 256-byte
 * aligned) for rows of S tokens.  Host only: enqueues nothing. */
PBA_API int pba_map_init(pba_block_map* map, void* buffer, size_t buffer_bytes,
                 int B, int S, int block_m, int block_n);

/* Build the map from n_packs descriptors `packs` (device array of pba_pack)
 * and n_resp_total response lengths `resp_len` (device int32).  Validates
 * the descriptor contents on the device (map->status), then writes every
 * other field of the map (left unspecified when the status is not OK).
 * Asynchronous on `stream`. */
PBA_API int pba_pack_block_map(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                       const pba_block_map* map, void* stream);

/* The same for n_maps maps of the same rows (same B and S, any tile shapes;
 * `maps` is a host array of n_maps initialised maps, 1 <= n_maps <=
 * PBA_MAX_MAPS_PER_BUILD), built together in two launches (three when one side
 * of a map has more than 2048 tiles): the forward /
 * dQ map and the dK / dV map of a batch are built with one call.  Each map
 * ends up exactly as pba_pack_block_map would build it. */
#define PBA_MAX_MAPS_PER_BUILD 4
PBA_API int pba_pack_block_maps(const pba_pack* packs, int n_packs, const int32_t* resp_len, int n_resp_total,
                                const pba_block_map* maps, int n_maps, void* stream);

/* Aligned position ids, log-prob gather rows and the response loss mask of
 * a packed batch ("DPO Preference Packing: Dense Masks and Sparse
 * Execution", section "Layout requirements": response tokens keep the
 * position ids of their own prompt + response sequence, and log-probs are
 * gathered from the logits that predict each response token, a response's
 * first token from the final prompt row; "Pack training sequences to reduce
 * padding waste", sections on target boundaries and position IDs).
 * From a map built by pba_pack_block_map(s) (any tile shape), for token s
 * of row b (device arrays of B*S elements, caller-allocated; any of them
 * may be NULL and is then not written):
 *   pos_ids[b*S+s]   prompt token j -> j; token t of a response ->
 *                    prompt_len + t; 0 for pad
 *   src_row[b*S+s]   position in row b of the token whose logits predict
 *                    token s: s-1 inside a prompt or response, the last
 *                    prompt token for a response's first token, -1 when
 *                    there is none (a pack's first token, a response's
 *                    first token after an empty prompt, pad)
 *   loss_mask[b*S+s] 1 for a response token with src_row >= 0, else 0
 * Enqueued on `stream` after the map build; nothing is written when the
 * map's status is not OK.  Returns PBA_OK, PBA_ERR_NULL (map or its token
 * arrays), PBA_ERR_SHAPE or PBA_ERR_DEVICE. */
PBA_API int pba_pack_positions(const pba_block_map* map, int32_t* pos_ids, int32_t* src_row, uint8_t* loss_mask,
                               void* stream);

/* Packed token log-probs and per-response sums ("DPO Preference Packing:
 * Dense Masks and Sparse Execution", section "Layout requirements": a
 * response's log-prob is gathered from the logits that predict each of its
 * tokens, including the branch start).  With src_row and loss_mask from
 * pba_pack_positions on the same map, for every token t = b*S+s:
 *   tok_logp[t] = logits[b, src_row[t], y] - log sum_v exp(logits[b, src_row[t], v]),
 *                 y = tokens[t], where loss_mask[t] = 1; 0 where it is 0;
 *                 NaN when y is outside [0, V)
 * (fp32 accumulation), and, if resp_logp is not NULL, for every response i
 * of the descriptors (indexed like resp_len), resp_logp[i] = the sum of
 * tok_logp over its tokens in token order (deterministic).
 * logits: bf16 [B, S, V] device, 16-byte aligned, V a multiple of 8;
 * tokens int32 [B*S]; tok_logp fp32 [B*S]; resp_logp fp32 [n_resp_total];
 * packs / resp_len as given to the map build (needed only for resp_logp).
 * Enqueued on `stream`; nothing is written when the map's status is not OK.
 * Returns PBA_OK, PBA_ERR_NULL, PBA_ERR_SHAPE (B, S, V or counts),
 * PBA_ERR_ALIGN or PBA_ERR_DEVICE. */
PBA_API int pba_packed_token_logp(const pba_block_map* map, const pba_pack* packs, int n_packs,
                                  const int32_t* resp_len, int n_resp_total, const int32_t* src_row,
                                  const uint8_t* loss_mask, const void* logits, int V, const int32_t* tokens,
                                  float* tok_logp, float* resp_logp, void* stream);

/* Rotary embedding at the packed, branch-aligned position ids ("DPO
 * Preference Packing: Dense Masks and Sparse Execution", section "Layout
 * requirements": every response keeps the positions of its own
 * [prompt | response] sequence; the ids are those pba_pack_positions writes,
 * pad tokens 0).  For every token t and head h of x (bf16 [B, S, H, D],
 * device, 16-byte aligned; y the same shape, may be x itself):
 *   y[t,h,i]       = x[t,h,i] cos(a) - x[t,h,i+D/2] sin(a)
 *   y[t,h,i+D/2]   = x[t,h,i] sin(a) + x[t,h,i+D/2] cos(a),   i < D/2,
 *   a = pos(t) * base^(-2i/D), negated when inverse != 0
 * (rotate-half pairing; the inverse is the transpose rotation, which maps
 * gradients with respect to the rotated tensor to gradients with respect to
 * x).  Angles and products in fp32, output rounded to bf16.  Map from
 * pba_pack_block_map(s) for (B, S) (any tile shape); nothing is written when
 * its status is not OK.  Apply it to Q (H = Hq) and K (H = Hkv) before the
 * forward, and with inverse = 1 to dQ and dK after the backward.  Returns
 * PBA_OK, PBA_ERR_NULL, PBA_ERR_SHAPE, PBA_ERR_HEAD_DIM (D not 64 or 128),
 * PBA_ERR_ARG (base not above 1 and finite), PBA_ERR_ALIGN or
 * PBA_ERR_DEVICE. */
PBA_API int pba_packed_rope(const pba_block_map* map, const void* x, void* y, int H, int D, float base, int inverse,
                            void* stream);

/* Group preference objectives and their surrogate coefficients ("GroupDPO"
 * page, section "core formulas").  A batch holds n_groups groups in CSR
 * form: group g owns entries [group_ptr[g], group_ptr[g+1]); entry e names
 * response member[e] and is a positive (positive[e] != 0) or a negative.
 * Each group needs at least one of each and names a response at most once;
 * a response may belong to several groups.  From the per-response log-prob
 * sums of the policy and of the frozen reference (pol, ref: fp32 [n_resp],
 * e.g. resp_logp of pba_packed_token_logp) and the response lengths
 * (resp_len, int32 [n_resp], the same array as for the map build):
 *   u_i      = beta (pol_i / len_i - ref_i / len_i)
 *   loss[0]  = L_group = (1/n_groups) sum_g phi_g(u[P_g], u[N_g])
 *   coef[i]  = (1/n_groups) sum_{g containing i} d phi_g / d u_i
 *              (L_sur = sum_i coef_i u_i has the first-order gradient of
 *              L_group at this point; 0 for a response in no group)
 *   nll_w[i] = alpha sum_{g: i in P_g} 1 / (n_groups |P_g|), the weight of
 *              response i's mean token NLL in the positive-NLL term
 *   loss[1]  = alpha (1/n_groups) sum_g mean_{i in P_g} (-pol_i / len_i)
 * where phi is selected by `objective` (each is -log sigmoid(u+ - u-) for
 * one positive and one negative):
 *   PBA_GROUP_ALL_PAIRS  mean over (i in P, j in N) of -log sigmoid(u_i - u_j)
 *   PBA_GROUP_MARGIN     -log sigmoid(mean_P u - mean_N u)
 *   PBA_GROUP_MPO        log sum_{P u N} e^u - log sum_P e^u
 *   PBA_GROUP_SOFTMAX    mean over i in P of log(e^{u_i} + sum_N e^u) - u_i
 * Computed in fp64 by one workgroup, every sum in a fixed order
 * (deterministic); outputs rounded to fp32.  All arrays are device memory:
 * group_ptr int32 [n_groups+1], member int32 / positive uint8 [n_entries],
 * coef fp32 [n_resp], nll_w fp32 [n_resp] (may be NULL), loss fp32 [2]
 * (may be NULL), status int32 [2] = {PBA_GROUP_* code or 0, first bad group
 * or 0}.  Group contents are checked on the device: on a bad group, status
 * is set and coef, nll_w and loss are filled with NaN.  Limits: 2 <=
 * n_entries <= PBA_GROUP_MAX_ENTRIES, 1 <= n_groups <= n_entries / 2,
 * n_resp >= 1.  Returns PBA_OK, PBA_ERR_NULL, PBA_ERR_SHAPE, PBA_ERR_ARG
 * (objective unknown, beta not positive and finite, alpha negative or not
 * finite) or PBA_ERR_DEVICE. */
#define PBA_GROUP_ALL_PAIRS 0
#define PBA_GROUP_MARGIN    1
#define PBA_GROUP_MPO       2
#define PBA_GROUP_SOFTMAX   3
#define PBA_GROUP_MAX_ENTRIES 4096
PBA_API int pba_group_coefficients(const int32_t* group_ptr, int n_groups, const int32_t* member,
                                   const uint8_t* positive, int n_entries, const float* pol, const float* ref,
                                   const int32_t* resp_len, int n_resp, int objective, float beta, float alpha,
                                   float* coef, float* nll_w, float* loss, int32_t* status, void* stream);

/* Forward.  For every query token and q head: O = softmax(scale * Q K^T
 * restricted to the allowed keys) V, and LSE = natural log of the sum of
 * exp(scale * q.k) over the allowed keys (the softmax normaliser, kept for
 * the backward).  q, k, v, o: bf16 device arrays in the layouts above;
 * lse: fp32 [B, Hq, S].  Only the map's full and partial tiles are
 * computed; the mask is applied on partial tiles only.  The map must have
 * been built for (B, S) with the tile shape of pba_fwd_tile.  softmax_scale
 * must be positive and finite (PBA_ERR_SCALE).  One batch row of Q must be
 * under 2 GiB (S * Hq * D * 2 < 2^31, else PBA_ERR_SHAPE). */
PBA_API int pba_packed_attn_fwd(const pba_block_map* map, const void* q, const void* k, const void* v,
                        void* o, float* lse, int B, int S, int Hq, int Hkv, int D,
                        float softmax_scale, void* stream);

/* Forward for rotary inputs, with the rotation of Q fused in: q is the
 * UNROTATED Q, k_rot is K rotated by pba_packed_rope at the packed
 * positions with the same base.  Each workgroup rotates its Q block in
 * registers at the queries' packed positions before the scores (rotate-half
 * pairing; angles reduced to revolutions in fp32 for the hardware sine and
 * cosine) and, if q_rot is not NULL (bf16, Q's layout), also writes the
 * rotated Q there, which is what pba_packed_attn_bwd_rope takes.  O and LSE
 * as pba_packed_attn_fwd on the rotated inputs.  rope_base must be above 1
 * and finite (PBA_ERR_ARG). */
PBA_API int pba_packed_attn_fwd_rope(const pba_block_map* map, const void* q, const void* k_rot, const void* v,
                                     void* o, float* lse, void* q_rot, int B, int S, int Hq, int Hkv, int D,
                                     float softmax_scale, float rope_base, void* stream);

/* Workspace bytes the backward needs: two fp32 [B, Hq, S] arrays (minus the
 * row dot products rowsum(dO * O), and minus LSE / softmax_scale), written
 * by the dQ stage and read by the dK / dV stage, then the area of the dK / dV stage's
 * split key tiles (a key tile whose visit list is longer than the average
 * load of one workgroup slot is shared by two workgroups): arrival counters
 * and fp32 partial sums for at most min(256, B * ceil(S / 128) * Hq)
 * (key tile, kv head) pairs, 256 KB each at D = 128 (64 MB at most); 0 on
 * bad arguments. */
PBA_API size_t pba_bwd_workspace_bytes(int B, int S, int Hq, int D);

/* Backward of the forward above for the loss <dO, O>: dQ, dK, dV (bf16),
 * with dK / dV summed over the q heads that share a kv head.  o and lse are
 * the forward's outputs; dout is dO.  Two maps of the same descriptors:
 * qmap with the tile shape of pba_fwd_tile (the dQ stage walks query tiles)
 * and kmap with the tile shape of pba_bwd_tile (the dK / dV stage walks key
 * tiles).  workspace: device memory of at least pba_bwd_workspace_bytes,
 * 256-byte aligned, contents irrelevant (overwritten).  Every output
 * element is written exactly once (no accumulation into the outputs); the
 * two fp32 partial sums of a split key tile are added by whichever of its
 * two workgroups finishes second (an arrival counter decides), and a + b is
 * b + a, so the result is deterministic.  Calls that overlap on one
 * workspace race.  softmax_scale > 0. */
PBA_API int pba_packed_attn_bwd(const pba_block_map* qmap, const pba_block_map* kmap, const void* q, const void* k,
                                const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                                void* dv, void* workspace, size_t workspace_bytes, int B, int S, int Hq, int Hkv,
                                int D, float softmax_scale, void* stream);

/* The backward in its two stages, for callers that schedule or time them
 * separately.  `stages` is a bit mask; running both in order on one stream
 * is exactly pba_packed_attn_bwd:
 *   PBA_BWD_DQ    dQ written; workspace <- -rowsum(dO * O) and -LSE / scale
 *   PBA_BWD_DKDV  dK, dV written (reads the workspace the dQ stage wrote)
 * Arguments as for pba_packed_attn_bwd (all are checked for every stage);
 * returns PBA_ERR_SHAPE for an empty or unknown mask. */
#define PBA_BWD_DQ   1
#define PBA_BWD_DKDV 2
#define PBA_BWD_ALL  3
PBA_API int pba_packed_attn_bwd_stages(int stages, const pba_block_map* qmap, const pba_block_map* kmap,
                                       const void* q, const void* k, const void* v, const void* o, const float* lse,
                                       const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, int B, int S, int Hq, int Hkv, int D,
                                       float softmax_scale, void* stream);

/* Backward without allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  pba_packed_attn_bwd (both stages) with the caller's
 * workspace replaced by a scratch array the library keeps in device memory:
 * PBA_NOALLOC_SCRATCH_BYTES (96 MiB) on every device the library is used on,
 * held from the library's load until the process ends.  The call itself
 * allocates and frees nothing.  Arguments, results and errors are those of
 * pba_packed_attn_bwd without the workspace, plus PBA_ERR_SCRATCH when the
 * row statistics (two fp32 [B, Hq, S] arrays, i.e. 8 * B * Hq * S bytes,
 * and one counter) do not fit the scratch.  The rest of the scratch holds
 * the split key tiles' partial sums (256 KB per (key tile, kv head) pair at
 * D = 128): when fewer pairs fit than pba_bwd_workspace_bytes provides
 * for, fewer key tiles may be split, which changes only the rounding of
 * their dK / dV; otherwise the results are bit-identical to
 * pba_packed_attn_bwd's.  Every call on a device shares that device's
 * scratch and finds it as the last call left it (the kernels overwrite or
 * reset everything they read): calls that overlap on one device (two
 * streams, or two threads on one stream without ordering) race. */
#define PBA_NOALLOC_SCRATCH_BYTES (96u << 20)
PBA_API int pba_packed_attn_bwd_noalloc(const pba_block_map* qmap, const pba_block_map* kmap, const void* q,
                                        const void* k, const void* v, const void* o, const float* lse,
                                        const void* dout, void* dq, void* dk, void* dv, int B, int S, int Hq,
                                        int Hkv, int D, float softmax_scale, void* stream);

/* Rounding of dK / dV and the compute-unit count.  A key tile whose visit
 * list is longer than 1.05 times the average load of one workgroup slot
 * (all visited tiles of kmap over `slots`, the slots per kv group) is
 * split between two workgroups; its dK / dV are then the sum of two fp32
 * partial sums, one per half of its list, instead of one running sum.  By
 * default slots = compute units of the device / Hkv, so which tiles are
 * split, and with it the last bits of their dK / dV, depends on the device's
 * CU count: results are bit-identical from run to run on one device (and
 * across devices with the same count) but may differ in rounding between
 * devices or partition modes with different counts (both stay within the
 * same error bound of exact arithmetic).  pba_set_bwd_split_slots(n) fixes
 * slots = n for every later backward call of this process (n >= 1), or
 * restores the default (n = 0), and returns the previous setting (0 for
 * the default); PBA_ERR_SHAPE for n < 0.  Process-wide: set it before
 * calls are enqueued, not while another thread enqueues one. */
PBA_API int pba_set_bwd_split_slots(int slots);

/* Backward for rotary inputs, with the rotation of the gradients fused in.
 * q_rot, k_rot are Q and K rotated by pba_packed_rope at the packed
 * positions (with this base); o and lse come from pba_packed_attn_fwd on
 * them.  Writes dV and the gradients with respect to the UNROTATED Q and K
 * (dQ, dK rotated back at each token's packed position inside the kernels'
 * epilogues, in fp32 before the bf16 rounding), so no inverse rotation pass
 * is needed.  Everything else as pba_packed_attn_bwd; rope_base must be
 * above 1 and finite (PBA_ERR_ARG). */
PBA_API int pba_packed_attn_bwd_rope(const pba_block_map* qmap, const pba_block_map* kmap, const void* q_rot,
                                     const void* k_rot, const void* v, const void* o, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                     size_t workspace_bytes, int B, int S, int Hq, int Hkv, int D,
                                     float softmax_scale, float rope_base, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PBA_H */
