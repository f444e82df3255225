// LDS tile layout, transposing LDS reads and buffer resources shared by the
// prefill kernels (gfx950).
#pragma once

#include "la_common.h"

namespace la {

// ------------------------------------------------------------------ LDS tiles

// Row-major LDS tile of RL-element rows.  fp32 tiles are padded by one
// 16-byte vector per row.  bf16 tiles are unpadded; the 16-byte unit index of
// a row is XORed with a hash of the row number (bits r3..r0):
//   RL = 64  (8 units):  h = 4 r1 + 2 (r2 ^ r3) + r2
//   RL = 128 (16 units), 256 (32 units): h = 8 r1 + 4 r0 + 2 (r2 ^ r3) + r2
// With it, each of the access patterns below touches every LDS bank equally
// often per hardware pass: 16 consecutive rows at one 16-byte unit (row reads
// of phi(Q)/phi(K) and 8-byte state writes), rows {b..b+3, b+8..b+11} at 32
// contiguous bytes (transposing reads over k-steps), rows {b..b+7} at 32
// contiguous bytes (transposing reads of value blocks), and whole rows
// (staging writes).  An 8-byte piece never straddles a 16-byte unit, so the
// transposing reads see contiguous 4-element pieces.
template <typename OP, int RL>
struct Tile {
  static constexpr int kStride = sizeof(OP) == 2 ? RL : RL + 16 / (int)sizeof(OP);
  static constexpr int elems(int rows) { return rows * kStride; }
  __device__ static __forceinline__ int hash(int r) {
    if constexpr (RL == 64) {
      return (((r >> 1) & 1) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
    } else {
      // 128 or 256 elements per row: rows start at the same bank, and the
      // hash only permutes 16-byte units inside each 256-byte half row
      static_assert(RL == 128 || RL == 256, "bf16 tiles of 64, 128 or 256 elements per row");
      return (((r >> 1) & 1) << 3) | ((r & 1) << 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
    }
  }
  __device__ static __forceinline__ int off(int row, int col) {
    if constexpr (sizeof(OP) == 2) {
      return row * RL + ((((col >> 3) ^ hash(row)) << 3) | (col & 7));
    } else {
      return row * kStride + col;
    }
  }
};

// Buffer resource over [base, base + bytes): out-of-range loads return zero
// and out-of-range stores are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// A store offset that is past the end of every buffer the kernels address:
// the entry points refuse heads whose Q/K/V/O reach 2^31 bytes, and every
// supported row is at least 128 bytes, so a head buffer ends at or below
// 2^31 - 128 = 0x7fffff80.  Stores at kDropOffset - 16 i (i < 4) are
// dropped by the buffer range check.
constexpr int kDropOffset = 0x7ffffff0;

// Compiler-only ordering point: memory operations are not moved across it
// (no instruction is emitted).  Used where the issue order of loads decides
// how exactly the compiler can count outstanding memory operations.
__device__ __forceinline__ void mem_order_fence() { asm volatile("" ::: "memory"); }

// Cache policy of the output stores: nt (streaming).  O is written once and
// not read again by the path; with this policy its lines do not linger dirty
// in the memory-side cache, where the next kernel of a step (the next span
// state pass) would otherwise pay for their write-back while it reads K and V.
constexpr int kStreamStore = 2;
// The same policy on the output pass's Q loads (Q is read once): measured
// faster for the output kernel, while on the state pass's K and V loads it
// slows the output pass that re-reads them.
constexpr int kStreamLoad = 2;

// ------------------------------------------------------------------ LDS fragments

__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// bf16 operand fragment whose 8 k-slots run down two groups of 4 rows of a
// row-major LDS tile (slots 0-3: rows ra..ra+3, slots 4-7: rows rb..rb+3) at
// this lane's column col_base + li (lane li reads row ra + li/4 at column
// col_base + 4 (li%4)).
template <int RL>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* base, int ra, int rb, int col_base, int li) {
  using TL = Tile<bf16, RL>;
  const int col = col_base + 4 * (li & 3);
  const bf16x4 x = ds_read_tr4(base + TL::off(ra + (li >> 2), col));
  const bf16x4 y = ds_read_tr4(base + TL::off(rb + (li >> 2), col));
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same fragment with the upper 4 slots zero (a 16-token chunk).
template <int RL>
__device__ __forceinline__ bf16x8 tr_frag_lo(const bf16* base, int ra, int col_base, int li) {
  using TL = Tile<bf16, RL>;
  const bf16x4 x = ds_read_tr4(base + TL::off(ra + (li >> 2), col_base + 4 * (li & 3)));
  const bf16x4 z4 = bf16x4{0, 0, 0, 0};
  return __builtin_shufflevector(x, z4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Buffer resources of one head's Q, K (N x D) and V, O (N x DV).
struct HeadBufs {
  __amdgpu_buffer_rsrc_t q, k, v, o;
  __amdgpu_buffer_rsrc_t a;  // per-token log gates of the head (gated decay only)
};

}  // namespace la
