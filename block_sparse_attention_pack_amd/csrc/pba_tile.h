// Device helpers for the attention kernels: MFMA wrappers, LDS transpose
// reads, bf16 packing.  Lane layouts (wave64, verified on gfx950):
//   v_mfma_f32_32x32x16_bf16:  A[i][k]: lane l holds i = l%32, k = 8*(l/32)+0..7
//                              B[k][j]: lane l holds j = l%32, k = 8*(l/32)+0..7
//                              C[i][j]: lane l, register r holds
//                                       j = l%32, i = 8*(r/4) + 4*(l/32) + r%4
//   ds_read_b64_tr_b16: in each group of 16 lanes, source lane s addresses 4
//     consecutive 16-bit elements; destination lane i receives element i%4
//     of source lanes i/4, 4+i/4, 8+i/4, 12+i/4.  If source lane s points at
//     M[r0 + s/4][c0 + 4*(s%4)] of a row-major matrix M, lane i receives
//     M[r0 + t][c0 + i] for t = 0..3: a 4 x 16 block read column-wise.
#pragma once
#include <type_traits>

#include "pba_internal.h"

namespace pba {

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PBA_LDS i16x4*)((PBA_LDS char*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// 8 values for a 32x32x16 operand whose k index runs down the rows of a
// row-major LDS matrix M (row stride `stride` elements):
// lane l gets M[rows(t)][col0 + 16*((l/16)%2) + l%16] where rows(t) = r0 + t
// for t < 4 and r1 + t - 4 for t >= 4 (r0, r1 already include the lane's
// 4*(l/32) offset chosen by the caller).
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* M, int stride, int r0, int r1, int col0, int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int col = col0 + 16 * (G & 1) + 4 * (s & 3);
  const bf16x4 lo = lds_tr4(M + (r0 + (s >> 2)) * stride + col);
  const bf16x4 hi = lds_tr4(M + (r1 + (s >> 2)) * stride + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS row permutation used by every staged tile (rows of D + 8 elements):
// inside each group of 16 rows, row 4j + i is stored at 4i + j (a 4 x 4
// transpose; its own inverse).  With that padding, the 16 rows an A-operand
// load reads together still fall in 16 different bank groups, and the 4
// consecutive rows of a transpose read land 4 bank groups apart, so neither
// access conflicts (both conflict without the permutation).  Addresses stay
// additive in the compile-time parts, so no extra registers are needed.
__device__ __forceinline__ int prow(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// Visibility of the 64 keys jb + off (off = 0..63) of a partial tile to one
// query, as a bit mask (bit off of the pair {lo word, hi word}).  The query
// sees its pack's shared prompt up to the end of the prompt and its own
// branch up to itself: with lim = q - jb, the branch run starting at
// lo = kv_lo - jb and the prompt run [-pc, plen - pc) (pc = jb - pre_lo,
// plen = pre_hi - pre_lo), key off is visible iff off <= lim and it lies in
// either run.  Built once per tile; then a score needs one bit extract.
struct KeyMask {
  unsigned lo, hi;
};
__host__ __device__ __forceinline__ unsigned long long key_run_bits(int a, int b) {
  // bits [a, b) of 0..63
  a = a < 0 ? 0 : a;
  b = b > 64 ? 64 : b;
  if (b <= a) return 0ull;
  return (~0ull << a) & (~0ull >> (64 - b));
}
__host__ __device__ __forceinline__ KeyMask key_mask(int lim, int lo, int pc, int plen) {
  const int end = lim + 1;
  const int pend = plen - pc < end ? plen - pc : end;
  const unsigned long long m = key_run_bits(lo, end) | key_run_bits(-pc, pend);
  return {(unsigned)m, (unsigned)(m >> 32)};
}
// Rotary embedding of an MFMA accumulator block in the transposed layout
// (lane: one token; register r of block e: head dim 32*e + 8*(r/4) + 4*hi +
// r%4), rotate-half pairing: dim d < D/2 pairs with d + D/2, i.e. block e
// with block e + NE/2 in the same lane and register.  The angle is
// sign * pos * base^(-2d/D), reduced to revolutions in fp32 before the
// hardware sine and cosine (which take revolutions).
template <int NE>
__device__ __forceinline__ void rope_rotate_t(f32x16 (&acc)[NE], int pos, int hi, float log2_base, float sign) {
  constexpr int D = 32 * NE;
  const float p = sign * (float)pos * 0.15915494309189535f;  // pos / (2 pi)
#pragma unroll
  for (int e = 0; e < NE / 2; ++e) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * e + 8 * (r >> 2) + 4 * hi + (r & 3);
      float rev = p * exp2f(-(float)(2 * d) / (float)D * log2_base);
      rev -= floorf(rev);
      const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
      const float u = acc[e][r], v = acc[e + NE / 2][r];
      acc[e][r] = u * cs - v * sn;
      acc[e + NE / 2][r] = u * sn + v * cs;
    }
  }
}

// All ones if bit `bit` (a constant after unrolling) of w is set, else 0
// (one bit-field extract).
__device__ __forceinline__ int mask_bit(unsigned w, int bit) { return __builtin_amdgcn_sbfe((int)w, bit, 1); }
// s where the mask word m is all ones, -inf where it is 0 (one bit-field
// insert).
__device__ __forceinline__ float keep_or_ninf(int m, float s) {
  return __int_as_float((__float_as_int(s) & m) | (int)(0xff800000u & ~(unsigned)m));
}
// p where m is all ones, 0 where it is 0.  m is made opaque first: the
// optimiser would otherwise turn the extract and the AND into a compare and
// a select (three instructions where two do).
__device__ __forceinline__ float keep_or_zero(int m, float p) {
  asm("" : "+v"(m));
  return __int_as_float(__float_as_int(p) & m);
}

// lds_tr8 on a tile stored with prow(): r0, r1 are multiples of 4.
__device__ __forceinline__ bf16x8 lds_tr8p(const bf16* M, int stride, int r0, int r1, int col0, int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int col = col0 + 16 * (G & 1) + 4 * (s & 3);
  const bf16x4 lo = lds_tr4(M + prow(r0 + (s >> 2)) * stride + col);
  const bf16x4 hi = lds_tr4(M + prow(r1 + (s >> 2)) * stride + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One direct buffer->LDS load: each lane fetches SIZE bytes (4 or 16) at
// byte offset voff of the resource and the wave writes them to LDS at
// lds_dst + SIZE * lane (lds_dst wave-uniform).  Issued as inline assembly
// so that the compiler does not attach its own completion waits to later
// LDS reads (it cannot tell which LDS range the load writes and would make
// every read wait for it).  The caller orders the load: it never reads the
// destination before an explicit wait_vmem() and a barrier, and never
// loads into a buffer that another wave may still be reading.
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rs, const void* lds_dst, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const unsigned m0 = (unsigned)(uintptr_t)(PBA_LDS const void*)lds_dst;
  if (SIZE == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                 "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
                 "s"(m0)
                 : "memory", "m0");
#endif
}

// Makes v opaque to the optimiser so that it stays in its own register for
// as long as it lives (used for the per-lane offsets of the tile loads, which
// would otherwise be recomputed before every load).
__device__ __forceinline__ void pin(int& v) { asm volatile("" : "+v"(v)); }

// p plus an offset of 0 that the optimiser cannot see through.
template <typename T>
__device__ __forceinline__ T* opaque_lds(T* p) {
  int z = 0;
  asm volatile("" : "+s"(z));
  return p + z;
}

// Read-only map arrays through the constant address space, so that
// wave-uniform indices become scalar loads (they then never wait behind the
// vector-memory counter that also tracks the tile loads).
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ cint_ptr cptr(const int32_t* p) { return (cint_ptr)p; }

// Buffer resource over `rows` rows of a bf16 array with rows of D elements
// every row_stride elements, starting at `base`.  Offsets past the last
// row's data read as zero (hardware range check on the per-lane offset).
// The host guarantees that a batch row of every tensor is under 2 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* base, int rows, int row_stride, int D) {
  const int nbytes = ((rows - 1) * row_stride + D) * 2;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nbytes, 0x00020000);
}

// Direct buffer->LDS staging of ROWS rows x D into an LDS tile with padded
// rows of STR elements, row r of the tile at LDS row prow(r), by a
// workgroup of NWAVES waves.  A wave instruction fills 1 KB of LDS in lane order,
// so lane L of instruction q owns LDS bytes 1024*q + 16*L; the row and chunk
// there decide which global chunk it fetches (lanes in a row's padding fetch
// that row's last chunk again; the padding is never read).  The per-lane
// offsets are fixed for the whole kernel; the tile's position goes into the
// (scalar) buffer resource, whose range ends at the last valid row, so rows
// past the end of the sequence read as zeros.
template <int D, int STR, int ROWS = 64, int NWAVES = 4>
struct Stager {
  static constexpr int NI = ROWS * STR * 2 / 1024;  // 1 KB instructions per tile
  static constexpr int PER_WAVE = (NI + NWAVES - 1) / NWAVES;
  static_assert((ROWS * STR * 2) % 1024 == 0, "tile must be whole 1 KB blocks");
  int off[PER_WAVE];  // byte offset of this lane's chunk from the tile's first row
  int w;
  int row_stride;

  __device__ __forceinline__ Stager(int tid, int row_stride_elems) : row_stride(row_stride_elems) {
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int chunk = 64 * (w * PER_WAVE + i) + lane;
      const int p = min(chunk / (STR / 8), ROWS - 1), c = min(chunk % (STR / 8), D / 8 - 1);
      off[i] = prow(p) * row_stride_elems * 2 + 16 * c;  // LDS row p holds tile row prow(p)
      pin(off[i]);
    }
  }
  // Rows [0, ROWS) of the tile starting at `tile`, of which `rows` (>= 1)
  // are valid, into lds_tile.
  // (The builtin exists only for the device; the host pass, which never runs
  // this, must not instantiate it or it drops the kernels' host stubs.)
  __device__ __forceinline__ void stage(bf16* lds_tile, const bf16* tile, int rows) const {
#if defined(__HIP_DEVICE_COMPILE__)
    stage_rs(lds_tile, rows_rsrc(tile, rows, row_stride, D));
#endif
  }
  // The same from a resource built by the caller (rows_rsrc of the tile).
#if defined(__HIP_DEVICE_COMPILE__)
  __device__ __forceinline__ void stage_rs(bf16* lds_tile, __amdgpu_buffer_rsrc_t rs) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = w * PER_WAVE + i;
      if (q < NI) dma_to_lds<16>(rs, lds_tile + 512 * q, off[i]);
    }
  }
#endif
};

// A workgroup's block of R rows x RB bytes that are contiguous within a row
// in HBM (e.g. one query tile's rows over the workgroup's adjacent heads),
// rows `row_bytes` apart, mirrored in LDS with rows padded by 16 bytes.
// Both directions move whole 16-byte chunks with consecutive lanes on
// consecutive addresses, so every wave instruction covers full row segments.
template <int R, int RB>
struct RowBlock {
  static_assert(RB % 16 == 0, "rows are whole 16-byte chunks");
  static constexpr int LSTR = RB + 16;            // LDS row stride (bytes)
  static constexpr int CH = LSTR / 16;            // chunks per LDS row, pad included
  static constexpr int NI = (R * CH + 63) / 64;   // DMA wave instructions for the block
  static constexpr int BYTES = NI * 1024;         // LDS bytes written by load()

  // HBM -> LDS with direct loads (wave w of NWAVES issues instructions
  // w, w + NWAVES, ...); rows >= rows_valid (>= 1) read as zeros.  The
  // caller waits (wait_vmem + barrier) before reading the block.
  template <int NWAVES>
  __device__ __forceinline__ static void load(char* lds, const void* g, int rows_valid, int row_bytes, int w,
                                              int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int nbytes = (rows_valid - 1) * row_bytes + RB;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)g, (short)0, nbytes, 0x00020000);
    for (int i = w; i < NI; i += NWAVES) {
      const int c = 64 * i + lane;
      const int p = min(c / CH, R - 1), cc = min(c % CH, RB / 16 - 1);
      dma_to_lds<16>(rs, lds + 1024 * i, p * row_bytes + 16 * cc);
    }
#endif
  }
  // LDS -> HBM by NT threads, rows >= rows_valid skipped.  The stores are
  // non-temporal: every caller stores an output block that its kernel does
  // not read again, and keeping those lines out of the caches leaves them to
  // the tiles that are re-read (whole step 564 -> 537 us at the
  // Qwen3-8B-shaped packs, even though the dQ kernel then reads O from
  // memory).
  template <int NT>
  __device__ __forceinline__ static void store(void* g, const char* lds, int rows_valid, int row_bytes, int tid) {
    constexpr int RC = RB / 16, TOTAL = R * RC;
#pragma unroll
    for (int i = 0; i < (TOTAL + NT - 1) / NT; ++i) {
      const int c = tid + NT * i;
      const int p = c / RC, cc = c % RC;
      if ((TOTAL % NT == 0 || c < TOTAL) && p < rows_valid)
        __builtin_nontemporal_store(*(const u32x4*)(lds + p * LSTR + 16 * cc),
                                    (u32x4*)((char*)g + (int64_t)p * row_bytes + 16 * cc));
    }
  }
};

// src[0..63] (fp32, of which the first n >= 1 are valid; the rest read as
// 0) straight into LDS dst[0..63], one value per lane; lane4 = 4 * lane,
// pinned by the caller.
__device__ __forceinline__ void buffer_lds_dword(const float* src, int n, float* dst, int lane4) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, n * 4, 0x00020000);
  dma_to_lds<4>(rs, dst, lane4);
#endif
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
// (hand-scheduled sequences index registers by I, which must be constant).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// Keeps the instruction scheduler from moving anything across this point
// (used between the phases of a tile so that operand loads of a later
// phase are not hoisted, which would cost registers).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (bf16)x[base + t];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_half_swap(float x) { return __shfl_xor(x, 32); }

// max(x of this lane, x of lane ^ 32) with one VALU permute (no LDS trip):
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, so afterwards {a, b} hold both halves' values
// in every lane.
__device__ __forceinline__ float half_max(float x) {
  float a = x, b = x;
  asm volatile("v_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pba
