// Shared definitions of the HIP path (device and host).  Not part of the
// public ABI: the packed layout and the launch structures are internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbf {

typedef _Float16 half_t;
typedef half_t v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Global-address-space views: loads through these compile to global_load
// (tracked by vmcnt alone) instead of flat loads.
#define DBF_GLOBAL __attribute__((address_space(1)))
typedef const DBF_GLOBAL uint32_t* gu32p;
typedef const DBF_GLOBAL v8i* gv8ip;
typedef const DBF_GLOBAL v4u* gv4up;

// ---------------------------------------------------------------------------
// Packed sign layout (one bit per sign; bit value 1 means -1).
//
// A rows x cols sign matrix is packed along cols (the reduction dimension of
// its product).  Rows form tiles of 16 and quads of 4 tiles (64 rows); cols
// form blocks of 128.  Each (row quad, col block) unit is 1 KB, units stored
// quad-major: unit (rq, kb) starts at word (rq * nkb + kb) * 256.  Inside a
// unit, lane lam (0..63) owns 4 consecutive words, one per row tile h of the
// quad: word lam*4 + h holds row rho = lam % 16 of tile 4*rq + h.  With lane
// group g = lam / 16, slot s = 0..31 of the word is col
//     kb*128 + slot_col(g, s),   slot_col(g, s) = 32*(s/8) + 8*g + s%8,
// i.e. the two 2-bit fields of the block-local col index are (s/8, g).  One
// 16-byte load per lane brings four row tiles' words for one col block, and
// a wave's load is 1 KB contiguous.  The col order makes the eight slots
// 8j..8j+7 of the four lane groups one contiguous run of 32 cols, so the
// activations that meet them are read 64 bytes at a time per token.
// Inside a word, slot s sits at bit
//     b(s) = 4 * (s % 8) + s / 8
// so that slots 8d..8d+7 occupy bits d, d+4, ..., d+28.  This order lets a
// lane turn a word into fp4 operands with a shift and a mask per register:
// ((w << (3-d)) & 0x88888888) | 0x22222222 is +-1.0 in e2m1 for 8 slots.
// Padding rows and cols are +1 (bit 0).
constexpr int kRowTile = 16;
constexpr int kQuad = 4;
constexpr int kColBlock = 128;
constexpr int kUnitWords = 256;

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int slot_bit(int s) { return 4 * (s & 7) + (s >> 3); }
// block-local col of slot s in a word of lane group g (see above)
__host__ __device__ inline int slot_col(int g, int s) { return 32 * (s >> 3) + 8 * g + (s & 7); }
// word of (row tile rt, col block kb, lane lam) in a matrix with nkb col blocks
__host__ __device__ inline int64_t packed_word(int64_t rt, int64_t kb, int lam, int64_t nkb) {
  return ((rt >> 2) * nkb + kb) * kUnitWords + lam * 4 + (rt & 3);
}
__host__ __device__ inline int64_t packed_words_total(int64_t rows, int64_t cols) {
  return cdiv(rows, kRowTile * kQuad) * cdiv(cols, kColBlock) * kUnitWords;
}

// One adapter's factors (device pointers).
struct Factors {
  const uint32_t* B1;
  const uint32_t* B2;
  const half_t* alpha;
  const half_t* beta;
  const half_t* gamma;
};

// A run of consecutive tokens [t0, t1) served by one adapter (adapter < 0:
// tokens that contribute nothing).
struct ColBlock {
  int32_t t0, t1, adapter, pad;
};

// Workspace header written by the segmentation kernel.
struct WsHeader {
  int32_t n_colblocks;
  int32_t pad[63];
};

}  // namespace dbf
