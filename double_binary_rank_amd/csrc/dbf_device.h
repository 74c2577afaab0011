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

// A operand of v_mfma_f32_16x16x32_f16 for step s of a 128-block (k = 32s +
// 8g + e, e = 0..7, lane group g) from a lane's packed word w: ((w << (3-s))
// & 0x88888888) | 0x22222222 holds the 8 signs of the step as e2m1 +-1.0
// (slot 8s+e sits at bit 4e+s), and four v_cvt_scalef32_pk_f16_fp4 turn its
// bytes into f16 pairs.  msk = 0x88888888 and one = 0x22222222 are passed in
// registers.
template <int s>
__device__ inline v8h expand_cvt(uint32_t w, uint32_t msk, uint32_t one) {
  const uint32_t n = and_or(w << (3 - s), msk, one);
  const v2h r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n, 1.0f, 0);
  const v2h r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n, 1.0f, 1);
  const v2h r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n, 1.0f, 2);
  const v2h r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(n, 1.0f, 3);
  return v8h{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Issues one 16-byte-per-lane direct-to-LDS load: lane L's 16 bytes at
// base + voff go to LDS byte address lds + 16*L.  Written as inline asm so
// that the compiler does not order every later LDS read after it (it cannot
// tell which LDS bytes the load writes); the kernel waits for these loads
// itself with s_waitcnt on vmcnt before the barrier that publishes them.
// M0 (the LDS address operand) is saved and restored around the load.
__device__ inline void dma16(const void* base_, uint32_t voff, uint32_t lds_) {
  // base and lds are wave-uniform: pin them to scalar registers
  const uint64_t bu = (uint64_t)(uintptr_t)base_;
  // (readfirstlane returns a signed int: widen each half as unsigned)
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bu >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bu);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}

// As dma16 with 4 bytes per lane (lane L's 4 bytes go to lds + 4*L).
__device__ inline void dma4(const void* base_, uint32_t voff, uint32_t lds_) {
  const uint64_t bu = (uint64_t)(uintptr_t)base_;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bu >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bu);
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_);
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}

// s_waitcnt with vmcnt <= n only (expcnt and lgkmcnt at their maximum).
template <int n>
__device__ inline void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with vmcnt <= n and lgkmcnt = 0 (every LDS read returned).
template <int n>
__device__ inline void wait_vm_lds() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
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

// As segment_runs for T <= 64 * NW * PER, in one pass: thread j takes the
// PER consecutive tokens from PER * j, and every id is requested at once.
// A token's run start is the last run start at or before it: within the
// wave, the nearest lower lane with a run start (a ballot and one shuffle
// that every lane takes part in);
// across waves, the last run start of the waves before (LDS).  A thread's
// block-start count (0..PER, under 16) goes to the other lanes bit by bit
// through four ballots, and across waves through LDS.  Two barriers.
template <int NW, int PER, typename OnStart, typename OnEnd>
__device__ inline int32_t segment_runs_local(const int32_t* __restrict__ ids, int32_t T,
                                             int32_t n_adapters, int32_t chunk,
                                             OnStart&& on_start, OnEnd&& on_end) {
  static_assert(PER < 16, "block-start counts in four bits");
  __shared__ int32_t s_rs[NW];   // per wave: its last run start, -1 if none
  __shared__ int32_t s_cnt[NW];  // per wave: its block starts
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t tb = tid * PER;
  int32_t raw[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) raw[k] = tb + k < T ? ids[tb + k] : -1;
  const int32_t raw_prv = (tb >= 1 && tb - 1 < T) ? ids[tb - 1] : -1;
  int32_t id[PER];
  uint32_t rsb = 0;  // bit k: token tb + k starts a run
  int32_t my_last = -1;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    id[k] = tb + k < T ? norm_id(raw[k], n_adapters) : -1;
    const int32_t prv = k == 0 ? norm_id(raw_prv, n_adapters) : id[k - 1];
    if (tb + k < T && (tb + k == 0 || prv != id[k])) {
      rsb |= 1u << k;
      my_last = tb + k;
    }
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  const uint64_t H = __ballot(my_last >= 0);
  const int32_t wave_last = H ? __builtin_amdgcn_readlane(my_last, 63 - __clzll(H)) : -1;
  if (lane == 0) s_rs[w] = wave_last;
  __syncthreads();
  int32_t carry_rs = -1;
  for (int v = 0; v < w; ++v)
    if (s_rs[v] >= 0) carry_rs = s_rs[v];
  const uint64_t below = H & lt;
  const int src = below ? 63 - __clzll(below) : lane;
  const int32_t from_lane = __shfl(my_last, src);
  int32_t rs = below ? from_lane : carry_rs;  // run start before this thread's first token
  uint32_t bsb = 0;  // bit k: token tb + k starts a block
  int32_t cnt = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if ((rsb >> k) & 1u) rs = tb + k;
    if (tb + k < T && (tb + k - rs) % chunk == 0) {
      bsb |= 1u << k;
      ++cnt;
    }
  }
  int32_t before = 0, wtot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint64_t Bb = __ballot((cnt >> b) & 1);
    before += __popcll(Bb & lt) << b;
    wtot += __popcll(Bb) << b;
  }
  if (lane == 0) s_cnt[w] = wtot;
  __syncthreads();
  int32_t idx = before, total = 0;
  for (int v = 0; v < NW; ++v) {
    if (v < w) idx += s_cnt[v];
    total += s_cnt[v];
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if ((bsb >> k) & 1u) {
      on_start(idx, tb + k, id[k]);
      if (idx > 0) on_end(idx - 1, tb + k);
      ++idx;
    }
  }
  if (tid == 0 && total > 0) on_end(total - 1, T);
  return total;
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
