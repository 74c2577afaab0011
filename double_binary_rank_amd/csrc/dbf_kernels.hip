// HIP kernels for gfx950: sign packing and the path choice of the forward
// product.
//
// The product (LoRDBA summary, section 2 "Arquitectura Central"; DBF summary,
// section 2 "Calculo en la inferencia") is evaluated in two stages:
//   stage 1:  z_i[t][r] = beta_i[r] * sum_m S2[r][m] * (gamma_i[m] * x[t][m])
//   stage 2:  y[t][n]   = sum_i alpha_i[n] * sum_r S1[n][r] * z_i[t][r]
// z lives in the caller's workspace: fp32 [ell][T][ldz] on the small-T path
// (dbf_gemv.hip), fp16 on the large-T path (dbf_gemm.hip).
#include <climits>

#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

// ============================================================== packing ====

__global__ void k_pack(const void* __restrict__ src, int dtype, int64_t rows, int64_t cols,
                       int64_t ld, int64_t nkb, int64_t total_words, uint32_t* __restrict__ dst) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_words) return;
  const int64_t unit = gid / kUnitWords;
  const int w = (int)(gid % kUnitWords);
  const int lam = w >> 2, h = w & 3;
  const int64_t row = ((unit / nkb) * kQuad + h) * kRowTile + (lam & 15);
  const int64_t k0 = (unit % nkb) * kColBlock;
  uint32_t word = 0;
  if (row < rows) {
    const int64_t base = row * ld;
    for (int s = 0; s < 32; ++s) {
      const int64_t k = k0 + slot_col(lam >> 4, s);
      if (k >= cols) continue;
      bool neg;
      if (dtype == 1)
        neg = ((const int8_t*)src)[base + k] < 0;
      else if (dtype == 2)
        neg = (float)((const half_t*)src)[base + k] < 0.0f;  // -0 and NaN are not < 0
      else
        neg = ((const float*)src)[base + k] < 0.0f;
      word |= (uint32_t)neg << slot_bit(s);
    }
  }
  dst[gid] = word;
}

__global__ void k_unpack(const uint32_t* __restrict__ src, int64_t rows, int64_t cols, int64_t nkb,
                         int64_t total_words, int8_t* __restrict__ dst, int64_t ld) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_words) return;
  const int64_t unit = gid / kUnitWords;
  const int w = (int)(gid % kUnitWords);
  const int lam = w >> 2, h = w & 3;
  const int64_t row = ((unit / nkb) * kQuad + h) * kRowTile + (lam & 15);
  const int64_t k0 = (unit % nkb) * kColBlock;
  if (row >= rows) return;
  const uint32_t word = src[gid];
  for (int s = 0; s < 32; ++s) {
    const int64_t k = k0 + slot_col(lam >> 4, s);
    if (k >= cols) continue;
    dst[row * ld + k] = ((word >> slot_bit(s)) & 1u) ? (int8_t)-1 : (int8_t)1;
  }
}

// Packed words of the cols x rows transpose S^T, gathered bit by bit from the
// packed words of S (rows x cols): output word gid holds, for its row r'
// (a column of S) and 32 columns c' (rows of S), the bits of S[c'][r'].
// The transpose of the update, dW^T = sum_i diag(gamma_i) S2^T diag(beta_i)
// S1^T diag(alpha_i), is again a double-binary product with S2^T and S1^T
// as its sign matrices; the input gradient of the LoRDBA training pipeline's
// backward pass (summary section 2 "Pipeline de Entrenamiento", step 3) is
// that product applied to the output gradient.  Padding bits are 0 (+1).
__global__ void k_transpose(const uint32_t* __restrict__ src, int64_t rows, int64_t cols,
                            int64_t nkb_src, int64_t nkb_dst, int64_t total_words,
                            uint32_t* __restrict__ dst) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total_words) return;
  const int64_t unit = gid / kUnitWords;
  const int w = (int)(gid % kUnitWords);
  const int lam = w >> 2, h = w & 3;
  const int64_t drow = ((unit / nkb_dst) * kQuad + h) * kRowTile + (lam & 15);  // a column of S
  const int64_t k0 = (unit % nkb_dst) * kColBlock;
  uint32_t word = 0;
  if (drow < cols) {
    // where column drow of S sits inside each packed word of S
    const int c = (int)(drow % kColBlock);
    const int g = (c >> 3) & 3, ss = 8 * (c >> 5) + (c & 7);
    const int64_t ublk = drow / kColBlock;
    for (int s = 0; s < 32; ++s) {
      const int64_t srow = k0 + slot_col(lam >> 4, s);  // a row of S
      if (srow >= rows) continue;
      const int64_t sw = ((srow / (kQuad * kRowTile)) * nkb_src + ublk) * kUnitWords +
                         4 * (16 * g + (int)(srow % kRowTile)) + (int)((srow % (kQuad * kRowTile)) / kRowTile);
      word |= ((src[sw] >> slot_bit(ss)) & 1u) << slot_bit(s);
    }
  }
  dst[gid] = word;
}

hipError_t launch_transpose(const uint32_t* src, int64_t rows, int64_t cols, uint32_t* dst,
                            hipStream_t s) {
  const int64_t total = packed_words_total(cols, rows);
  hipLaunchKernelGGL(k_transpose, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, src, rows,
                     cols, cdiv(cols, kColBlock), cdiv(rows, kColBlock), total, dst);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       uint32_t* dst, hipStream_t s) {
  const int64_t nkb = cdiv(cols, kColBlock);
  const int64_t total = packed_words_total(rows, cols);
  const int64_t grid = cdiv(total, 256);
  hipLaunchKernelGGL(k_pack, dim3((unsigned)grid), dim3(256), 0, s, src, dtype, rows, cols, ld,
                     nkb, total, dst);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* src, int64_t rows, int64_t cols, int8_t* dst, int64_t ld,
                         hipStream_t s) {
  const int64_t nkb = cdiv(cols, kColBlock);
  const int64_t total = packed_words_total(rows, cols);
  const int64_t grid = cdiv(total, 256);
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)grid), dim3(256), 0, s, src, rows, cols, nkb, total,
                     dst, ld);
  return hipGetLastError();
}

// ============================================================ launching ====

size_t workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T) {
  return ws_layout(N, R, M, ell, T).total;
}

// The small-T path streams the signs once per column block of at most 5
// tokens; the large-T path costs a fixed few launches' latency, lowest when
// stage 1 reads x in place (a reduction of at most 8 blocks per wave, M <=
// 8192).  Whole calls replayed from graphs put the crossover at:
//   rank 64 (4096 x 4096): small-T faster through T = 12;
//   rank 2048 (4096 x 4096): large-T faster from T = 3;
//   rank 6368, 14336 x 4096: even at T = 2..5, large-T much faster from 6;
//   rank 6368, 4096 x 14336: small-T faster through T = 8, large-T at 12.
//   The multi-adapter call (whose large-T stage 1 never reads x in place)
//   keeps 16 tokens per segment as the switch, as measured on its batch.
Path choose_path(int64_t per_seg, int64_t R, int64_t M, bool multi) {
  if (multi || R < 256) return per_seg <= 16 ? Path::Gemv : Path::Mfma;
  if (per_seg <= 2) return Path::Gemv;
  if (M <= 8192) return Path::Mfma;
  return per_seg < 12 ? Path::Gemv : Path::Mfma;
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t s) {
  // small-T path: fp4 signs x 3-part fp8 activations on the scaled MFMA
  const int tcb = gemv_tokens_per_block(a.ell);
  if (tcb > 0 && a.T <= kGemvMaxT) {
    const int64_t segs = a.multi ? (a.num_adapters < a.T ? a.num_adapters : a.T) : 1;
    const int64_t per_seg = cdiv(a.T, segs);
    const bool want = a.path == Path::Gemv || (a.path != Path::Mfma && per_seg <= tcb);
    if (want) return launch_gemv(a, s);
  }
  // large-T path: fp16 matrix-core contractions
  return launch_gemm(a, s);
}

// Same-input layers: the grouped kernels run every layer in one launch per
// stage when the fast stages apply to all of them (the path launchers
// return hipErrorNotSupported, before launching anything, when they do
// not); otherwise the layers run one by one, each on its workspace slice.
hipError_t launch_forward_grouped(const ForwardArgs& a0, hipStream_t s) {
  ForwardArgs a = a0;
  a.single = a0.grp[0];
  hipError_t e = launch_forward(a, s);
  if (e != hipErrorNotSupported) return e;
  for (int j = 0; j < a0.group; ++j) {
    ForwardArgs b = a0;
    b.group = 0;
    b.single = a0.grp[j];
    b.y = (char*)a0.y + j * a0.y_layer_bytes;
    b.ws = (char*)a0.ws + j * a0.layer_ws;
    b.ws_bytes = a0.layer_ws;
    if ((e = launch_forward(b, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dbf
