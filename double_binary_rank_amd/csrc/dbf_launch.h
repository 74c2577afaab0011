// Launchers shared by the C-ABI layer and the kernels (internal).
#pragma once

#include "dbf_common.h"

namespace dbf {

// Which kernel family evaluates the two sign-accumulation stages.
enum class Path : int { Gemv = 0, Mfma = 1 };

struct ForwardArgs {
  // activations and output
  const half_t* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  bool y_f32;
  bool accumulate;
  // shapes
  int64_t N, R, M, T;
  int32_t ell;
  // factors: a single adapter, or device pointer tables + ids
  Factors single;
  bool multi;
  const int32_t* ids;
  int32_t num_adapters;
  const uint32_t* const* B1s;
  const uint32_t* const* B2s;
  const half_t* const* alphas;
  const half_t* const* betas;
  const half_t* const* gammas;
  // workspace
  void* ws;
  size_t ws_bytes;
  Path path;
};

size_t workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T);
hipError_t launch_pack(const void* src, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       uint32_t* dst, hipStream_t s);
hipError_t launch_unpack(const uint32_t* src, int64_t rows, int64_t cols, int8_t* dst, int64_t ld,
                         hipStream_t s);
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s);
Path choose_path(int64_t T, int64_t tokens_per_segment_estimate);

}  // namespace dbf
