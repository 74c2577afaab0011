// HIP kernels for gfx950: sign packing, the multi-adapter segmentation and
// the path choice of the forward product.
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

// ================================================== multi-adapter runs ====

// Splits the token sequence into runs of equal (normalised) adapter ids and
// each run into column blocks of at most `chunk` tokens.  One workgroup of
// 1024 threads walks the tokens in tiles of 1024 with two block-wide scans:
// a max-scan for the start of the run containing each token and a sum-scan
// over block starts for the output index.
__device__ inline int32_t norm_id(int32_t id, int32_t n) { return (id >= 0 && id < n) ? id : -1; }

__global__ __launch_bounds__(1024) void k_segment(const int32_t* __restrict__ ids, int64_t T,
                                                  int32_t num_adapters, int32_t chunk,
                                                  ColBlock* __restrict__ cbl,
                                                  WsHeader* __restrict__ hdr) {
  __shared__ int64_t s_max[1024];
  __shared__ int32_t s_sum[1024];
  __shared__ int64_t s_run_carry;
  __shared__ int32_t s_cnt_carry;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_run_carry = 0;
    s_cnt_carry = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < T; base += 1024) {
    const int64_t t = base + tid;
    const bool in = t < T;
    const int32_t id = in ? norm_id(ids[t], num_adapters) : -1;
    const bool run_start = in && (t == 0 || norm_id(ids[t - 1], num_adapters) != id);
    // max-scan: start of the run containing t
    s_max[tid] = run_start ? t : -1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int64_t v = tid >= off ? s_max[tid - off] : -1;
      __syncthreads();
      if (v > s_max[tid]) s_max[tid] = v;
      __syncthreads();
    }
    int64_t rs = s_max[tid];
    if (rs < 0) rs = s_run_carry;
    const bool blk_start = in && ((t - rs) % chunk == 0);
    // inclusive sum-scan of block starts
    s_sum[tid] = blk_start ? 1 : 0;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int32_t v = tid >= off ? s_sum[tid - off] : 0;
      __syncthreads();
      s_sum[tid] += v;
      __syncthreads();
    }
    if (blk_start) {
      const int32_t idx = s_cnt_carry + s_sum[tid] - 1;
      cbl[idx] = ColBlock{(int32_t)t, 0, id, 0};
    }
    __syncthreads();
    if (tid == 1023) {
      s_cnt_carry += s_sum[1023];
      s_run_carry = rs;
    }
    __syncthreads();
  }
  const int32_t n = s_cnt_carry;
  __syncthreads();
  for (int32_t j = tid; j < n; j += 1024) cbl[j].t1 = (j + 1 < n) ? cbl[j + 1].t0 : (int32_t)T;
  if (tid == 0) hdr->n_colblocks = n;
}

// ============================================================ launching ====

size_t workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T) {
  return ws_layout(N, R, M, ell, T).total;
}

Path choose_path(int64_t T, int64_t per_seg) {
  (void)T;
  return per_seg <= 16 ? Path::Gemv : Path::Mfma;
}

hipError_t launch_segment(const ForwardArgs& a, int chunk, hipStream_t s) {
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  hipLaunchKernelGGL(k_segment, dim3(1), dim3(1024), 0, s, a.ids, a.T, a.num_adapters, chunk,
                     (ColBlock*)(ws + L.cbl), (WsHeader*)ws);
  return hipGetLastError();
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

}  // namespace dbf
