// Device helpers shared by the stage kernels (internal).
#pragma once

#include "dbf_common.h"

namespace dbf {

typedef half_t v4h __attribute__((ext_vector_type(4)));
typedef half_t v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

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

__device__ inline int32_t norm_id(int32_t id, int32_t n) { return (id >= 0 && id < n) ? id : -1; }

// Column blocks of the multi-adapter paths: the maximal runs of tokens with
// equal adapter id (ids outside [0, n_adapters) count as -1 and form runs of
// their own, which the stage kernels skip), each cut into pieces of at most
// `chunk` tokens, numbered in token order.  Block idx covers tokens [t0, t1)
// of one adapter: on_start(idx, t0, adapter) and on_end(idx, t1) report it.
// Returns the number of blocks (the same in every thread).
//
// Run by ONE whole workgroup of 64*NW threads (every thread must call it),
// in passes of 64*NW ids.  Within a wave the start of a token's run and the
// rank of a block start come from ballots; the per-wave last run start and
// block count go through LDS (double-buffered by pass parity), so a pass has
// two barriers; the ids of the next pass are requested at the start of a
// pass.  The thread of a block start also ends the previous block.
template <int NW, typename OnStart, typename OnEnd>
__device__ inline int32_t segment_runs(const int32_t* __restrict__ ids, int32_t T,
                                       int32_t n_adapters, int32_t chunk, OnStart&& on_start,
                                       OnEnd&& on_end) {
  __shared__ int32_t s_last[2][NW];  // per wave: its last run start, -1 if none
  __shared__ int32_t s_cnt[2][NW];   // per wave: its block starts
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int32_t carry_rs = 0, carry_cnt = 0;  // equal in every thread
  int par = 0;
  int32_t nx_cur = tid < T ? ids[tid] : -1;
  int32_t nx_prv = (tid >= 1 && tid < T) ? ids[tid - 1] : -1;
  for (int32_t base = 0; base < T; base += 64 * NW, par ^= 1) {
    const int32_t t = base + tid;
    const bool in = t < T;
    const int32_t raw = nx_cur, raw_prv = nx_prv;
    const int32_t tn = t + 64 * NW;
    nx_cur = tn < T ? ids[tn] : -1;
    nx_prv = tn < T ? ids[tn - 1] : -1;
    const int32_t id = in ? norm_id(raw, n_adapters) : -1;
    const bool rstart = in && (t == 0 || norm_id(raw_prv, n_adapters) != id);
    const uint64_t M = __ballot(rstart);
    const int32_t wbase = base + 64 * w;
    if (lane == 0) s_last[par][w] = M ? wbase + 63 - __clzll(M) : -1;
    __syncthreads();
    // start of this token's run: the last run start at or before it
    const uint64_t upto = M & ((2ull << lane) - 1ull);  // lanes 0..lane
    int32_t rs = carry_rs;
    if (upto) {
      rs = wbase + 63 - __clzll(upto);
    } else {
      for (int v = 0; v < w; ++v)
        if (s_last[par][v] >= 0) rs = s_last[par][v];
    }
    const bool bstart = in && ((t - rs) % chunk == 0);
    const uint64_t B = __ballot(bstart);
    if (lane == 0) s_cnt[par][w] = __popcll(B);
    __syncthreads();
    int32_t idx = carry_cnt + __popcll(B & ((1ull << lane) - 1ull));
    for (int v = 0; v < w; ++v) idx += s_cnt[par][v];
    if (bstart) {
      on_start(idx, t, id);
      if (idx > 0) on_end(idx - 1, t);
    }
    for (int v = 0; v < NW; ++v) {
      if (s_last[par][v] >= 0) carry_rs = s_last[par][v];
      carry_cnt += s_cnt[par][v];
    }
  }
  if (tid == 0 && carry_cnt > 0) on_end(carry_cnt - 1, T);
  return carry_cnt;
}

// The column-block list in global memory (workgroup of 256 threads):
// cbl[idx] = {t0, t1, adapter, 0}, hdr->n_colblocks = count.
__device__ inline void segment_ids(const int32_t* __restrict__ ids, int32_t T, int32_t n_adapters,
                                   int32_t chunk, ColBlock* __restrict__ cbl,
                                   WsHeader* __restrict__ hdr) {
  const int32_t n = segment_runs<4>(
      ids, T, n_adapters, chunk,
      [&](int32_t idx, int32_t t, int32_t id) {
        cbl[idx].t0 = t;
        cbl[idx].adapter = id;
        cbl[idx].pad = 0;
      },
      [&](int32_t idx, int32_t t1) { cbl[idx].t1 = t1; });
  if (threadIdx.x == 0) hdr->n_colblocks = n;
}

}  // namespace dbf
