// Device helpers shared by the stage kernels (internal).
#pragma once

#include "dbf_common.h"

namespace dbf {

typedef half_t v4h __attribute__((ext_vector_type(4)));

// (a & m) | c in one VALU op (ALU only; no memory access).  gfx950 VOP3
// encodings take no literal constants, so m and c come from registers (m a
// wave-uniform SGPR, c a VGPR): the compiler would otherwise emit a separate
// and plus or with literals.
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

__device__ inline void store4(void* y, int64_t ldy, bool f32, int64_t t, int64_t r, int64_t rows,
                              const float v[4]) {
  if (f32) {
    float* p = (float*)y + t * ldy + r;
    if (r + 4 <= rows) {
      *(v4f*)p = v4f{v[0], v[1], v[2], v[3]};
    } else {
      for (int e = 0; e < 4; ++e)
        if (r + e < rows) p[e] = v[e];
    }
  } else {
    half_t* p = (half_t*)y + t * ldy + r;
    if (r + 4 <= rows) {
      *(v4h*)p = v4h{(half_t)v[0], (half_t)v[1], (half_t)v[2], (half_t)v[3]};
    } else {
      for (int e = 0; e < 4; ++e)
        if (r + e < rows) p[e] = (half_t)v[e];
    }
  }
}

__device__ inline void load4(const void* y, int64_t ldy, bool f32, int64_t t, int64_t r,
                             int64_t rows, float v[4]) {
  for (int e = 0; e < 4; ++e) {
    if (r + e < rows)
      v[e] = f32 ? ((const float*)y)[t * ldy + r + e] : (float)((const half_t*)y)[t * ldy + r + e];
    else
      v[e] = 0.0f;
  }
}

}  // namespace dbf
