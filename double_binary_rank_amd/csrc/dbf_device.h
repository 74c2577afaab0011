// Device helpers shared by the stage kernels (internal).
#pragma once

#include "dbf_common.h"

namespace dbf {

typedef half_t v4h __attribute__((ext_vector_type(4)));

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
