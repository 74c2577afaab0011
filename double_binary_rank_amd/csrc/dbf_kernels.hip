// HIP kernels for gfx950: sign packing, the two sign-accumulation stages and
// the multi-adapter segmentation.
//
// The product (LoRDBA summary, section 2 "Arquitectura Central"; DBF summary,
// section 2 "Calculo en la inferencia") is evaluated in two launches:
//   stage 1:  z_i[t][r] = beta_i[r] * sum_m S2[r][m] * (gamma_i[m] * x[t][m])
//   stage 2:  y[t][n]   = sum_i alpha_i[n] * sum_r S1[n][r] * z_i[t][r]
// z lives in the caller's workspace as fp32 [ell][T][ldz].
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
  const int64_t k0 = (unit % nkb) * kColBlock + 32 * (lam >> 4);
  uint32_t word = 0;
  if (row < rows) {
    const int64_t base = row * ld;
    for (int s = 0; s < 32; ++s) {
      const int64_t k = k0 + s;
      if (k >= cols) break;
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
  const int64_t k0 = (unit % nkb) * kColBlock + 32 * (lam >> 4);
  if (row >= rows) return;
  const uint32_t word = src[gid];
  for (int s = 0; s < 32; ++s) {
    const int64_t k = k0 + s;
    if (k >= cols) break;
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

// ===================================================== operand helpers ====

// Eight consecutive slots 8g..8g+7 of a packed word as fp16 +-1 (the A
// operand of v_mfma_f32_16x16x32_f16 for one lane).  With the packed bit
// order, slot 8g+2p sits at bit g+8p and slot 8g+2p+1 at bit g+8p+4.  After
// t = w >> g, a byte permute gathers bit 8p (via t << 7) into bit 15 and
// bit 8p+4 (via t << 3) into bit 31; the mask keeps those two sign bits and
// the constant supplies the magnitude 1.0 (0x3C00) in both halves.
__device__ inline v8h expand_signs_f16(uint32_t w, int g) {
  const uint32_t t = w >> g;
  const uint32_t U = t << 7, V = t << 3;
  v4u o;
  o[0] = (__builtin_amdgcn_perm(V, U, 0x040C000Cu) & 0x80008000u) | 0x3C003C00u;
  o[1] = (__builtin_amdgcn_perm(V, U, 0x050C010Cu) & 0x80008000u) | 0x3C003C00u;
  o[2] = (__builtin_amdgcn_perm(V, U, 0x060C020Cu) & 0x80008000u) | 0x3C003C00u;
  o[3] = (__builtin_amdgcn_perm(V, U, 0x070C030Cu) & 0x80008000u) | 0x3C003C00u;
  return __builtin_bit_cast(v8h, o);
}

// Stage-1 B operand: v = fp16(gamma[k+e] * x[k+e]), e = 0..7.  The fp16
// product is rounded once from the exact product (fp16 x fp16 fits fp32).
__device__ inline v8h act_stage1(const half_t* __restrict__ xrow, const half_t* __restrict__ g,
                                 int64_t k, int64_t K, bool valid, bool g_vec) {
  v8h r = {};
  if (!valid || k >= K) return r;
  if (k + 8 <= K) {
    const v8h xv = *(const v8h*)(xrow + k);
    v8h gv;
    if (g_vec) {
      gv = *(const v8h*)(g + k);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = g[k + e];
    }
    r = xv * gv;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e < K) r[e] = xrow[k + e] * g[k + e];
  }
  return r;
}

// Stage-2 B operand: z (fp32, workspace) rounded to fp16, masked past K.
__device__ inline v8h act_stage2(const float* __restrict__ zrow, int64_t k, int64_t K, bool valid) {
  v8h r = {};
  if (!valid || k >= K) return r;
  const v4f a = *(const v4f*)(zrow + k);
  const v4f b = *(const v4f*)(zrow + k + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (half_t)a[e];
    r[e + 4] = (half_t)b[e];
  }
  if (k + 8 > K) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e >= K) r[e] = (half_t)0.0f;
  }
  return r;
}

// ========================================================= stage kernel ====

struct StageParams {
  int64_t rows;   // output rows of this stage (R or N)
  int64_t K;      // reduction length (M or R)
  int64_t T;
  int32_t ell;
  int64_t nrt, nkb, nrb;
  const half_t* x;
  int64_t ldx;
  float* z;
  int64_t ldz, zstride;  // z_i[t][r] at z + i*zstride + t*ldz + r
  void* y;
  int64_t ldy;
  int32_t y_f32, accumulate;
  Factors single;
  int32_t multi;
  const ColBlock* cbl;
  const WsHeader* hdr;
  int64_t n_cb_host;
  int32_t num_adapters;
  const uint32_t* const* B1s;
  const uint32_t* const* B2s;
  const half_t* const* alphas;
  const half_t* const* betas;
  const half_t* const* gammas;
};

// Wave tile: (16*RW rows) x (16*CW tokens).  The four waves of a workgroup
// compute the same tile over four quarters of K and are summed in a fixed
// order through LDS (deterministic).  MFMA: A = signs (rows), B = activations
// (tokens); lane l holds D rows 4*(l/16)+v of token column l%16.
template <int STAGE, int RW, int CW>
__global__ __launch_bounds__(256) void k_stage_f16(StageParams p) {
  __shared__ float red[3][RW * CW * 4][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t n_cb = p.multi ? (int64_t)p.hdr->n_colblocks : p.n_cb_host;
  const int64_t n_items = n_cb * p.nrb;

  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t cb = it / p.nrb, rb = it % p.nrb;
    int64_t t0, t1;
    int32_t ad;
    Factors f;
    if (p.multi) {
      const ColBlock c = p.cbl[cb];
      t0 = c.t0;
      t1 = c.t1;
      ad = c.adapter;
      if (ad >= 0) {
        f.B1 = p.B1s[ad];
        f.B2 = p.B2s[ad];
        f.alpha = p.alphas[ad];
        f.beta = p.betas[ad];
        f.gamma = p.gammas[ad];
      }
    } else {
      t0 = cb * 16 * CW;
      t1 = t0 + 16 * CW < p.T ? t0 + 16 * CW : p.T;
      ad = 0;
      f = p.single;
    }
    const int64_t row0 = rb * 16 * RW;
    if (ad < 0) {
      // tokens routed to no adapter: zero their outputs (stage 2, overwrite mode)
      if (STAGE == 2 && !p.accumulate) {
        const int64_t nr = (p.rows - row0) < 16 * RW ? (p.rows - row0) : 16 * RW;
        for (int64_t e = threadIdx.x; e < (t1 - t0) * nr; e += blockDim.x) {
          const int64_t t = t0 + e / nr, r = row0 + e % nr;
          if (p.y_f32)
            ((float*)p.y)[t * p.ldy + r] = 0.0f;
          else
            ((half_t*)p.y)[t * p.ldy + r] = (half_t)0.0f;
        }
      }
      continue;
    }
    const uint32_t* __restrict__ S = STAGE == 1 ? f.B2 : f.B1;
    const int64_t kb0 = p.nkb * wv / 4, kb1 = p.nkb * (wv + 1) / 4;

    v4f yacc[RW][CW];
    if (STAGE == 2) {
#pragma unroll
      for (int rt = 0; rt < RW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CW; ++ct) yacc[rt][ct] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    for (int i = 0; i < p.ell; ++i) {
      v4f acc[RW][CW];
#pragma unroll
      for (int rt = 0; rt < RW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CW; ++ct) acc[rt][ct] = v4f{0.f, 0.f, 0.f, 0.f};
      const half_t* gi = STAGE == 1 ? f.gamma + (int64_t)i * p.K : nullptr;
      const bool g_vec = STAGE == 1 ? ((((uintptr_t)gi) & 15) == 0) : false;

      for (int64_t kb = kb0; kb < kb1; ++kb) {
        v4u wd[RW];
#pragma unroll
        for (int rt = 0; rt < RW; ++rt) {
          const int64_t tile = row0 / 16 + rt;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            wd[rt][q] = tile < p.nrt ? S[packed_word(tile, kb, 16 * q + c16, p.nkb)] : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t k = kb * kColBlock + 32 * q + 8 * g;
          v8h b[CW];
#pragma unroll
          for (int ct = 0; ct < CW; ++ct) {
            const int64_t t = t0 + ct * 16 + c16;
            const bool valid = t < t1;
            if (STAGE == 1)
              b[ct] = act_stage1(p.x + (valid ? t : 0) * p.ldx, gi, k, p.K, valid, g_vec);
            else
              b[ct] = act_stage2(p.z + i * p.zstride + (valid ? t : 0) * p.ldz, k, p.K, valid);
          }
#pragma unroll
          for (int rt = 0; rt < RW; ++rt) {
            const v8h a = expand_signs_f16(wd[rt][q], g);
#pragma unroll
            for (int ct = 0; ct < CW; ++ct)
              acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[ct], acc[rt][ct], 0, 0, 0);
          }
        }
      }

      // fixed-order cross-wave sum: wave 0 + wave 1 + wave 2 + wave 3
      if (wv > 0) {
#pragma unroll
        for (int rt = 0; rt < RW; ++rt)
#pragma unroll
          for (int ct = 0; ct < CW; ++ct)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wv - 1][(rt * CW + ct) * 4 + v][lane] = acc[rt][ct][v];
      }
      __syncthreads();
      if (wv == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
          for (int rt = 0; rt < RW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CW; ++ct)
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[rt][ct][v] += red[w][(rt * CW + ct) * 4 + v][lane];

        if (STAGE == 1) {
          const half_t* bi = f.beta + (int64_t)i * p.rows;
#pragma unroll
          for (int rt = 0; rt < RW; ++rt) {
            const int64_t r = row0 + rt * 16 + 4 * g;
            if (r >= p.rows) continue;
            float bs[4];
            for (int v = 0; v < 4; ++v) bs[v] = r + v < p.rows ? (float)bi[r + v] : 0.0f;
#pragma unroll
            for (int ct = 0; ct < CW; ++ct) {
              const int64_t t = t0 + ct * 16 + c16;
              if (t >= t1) continue;
              const float o[4] = {acc[rt][ct][0] * bs[0], acc[rt][ct][1] * bs[1],
                                  acc[rt][ct][2] * bs[2], acc[rt][ct][3] * bs[3]};
              store4(p.z + i * p.zstride, p.ldz, true, t, r, p.rows, o);
            }
          }
        } else {
          const half_t* ai = f.alpha + (int64_t)i * p.rows;
#pragma unroll
          for (int rt = 0; rt < RW; ++rt) {
            const int64_t r = row0 + rt * 16 + 4 * g;
            float as[4];
            for (int v = 0; v < 4; ++v) as[v] = r + v < p.rows ? (float)ai[r + v] : 0.0f;
#pragma unroll
            for (int ct = 0; ct < CW; ++ct)
#pragma unroll
              for (int v = 0; v < 4; ++v) yacc[rt][ct][v] += as[v] * acc[rt][ct][v];
          }
        }
      }
      __syncthreads();
    }

    if (STAGE == 2 && wv == 0) {
#pragma unroll
      for (int rt = 0; rt < RW; ++rt) {
        const int64_t r = row0 + rt * 16 + 4 * g;
        if (r >= p.rows) continue;
#pragma unroll
        for (int ct = 0; ct < CW; ++ct) {
          const int64_t t = t0 + ct * 16 + c16;
          if (t >= t1) continue;
          float o[4] = {yacc[rt][ct][0], yacc[rt][ct][1], yacc[rt][ct][2], yacc[rt][ct][3]};
          if (p.accumulate) {
            float old[4];
            load4(p.y, p.ldy, p.y_f32, t, r, p.rows, old);
            for (int v = 0; v < 4; ++v) o[v] += old[v];
          }
          store4(p.y, p.ldy, p.y_f32, t, r, p.rows, o);
        }
      }
    }
  }
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

template <int STAGE, int RW, int CW>
static hipError_t launch_stage(StageParams p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((k_stage_f16<STAGE, RW, CW>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int RW, int CW>
static hipError_t run_stages(StageParams p1, StageParams p2, bool multi, int64_t n_cb_max,
                             hipStream_t s) {
  p1.nrb = cdiv(p1.rows, 16 * RW);
  p2.nrb = cdiv(p2.rows, 16 * RW);
  int64_t g1 = n_cb_max * p1.nrb, g2 = n_cb_max * p2.nrb;
  if (multi) {
    g1 = g1 < 8192 ? g1 : 8192;
    g2 = g2 < 8192 ? g2 : 8192;
  }
  hipError_t e = launch_stage<1, RW, CW>(p1, g1, s);
  if (e != hipSuccess) return e;
  return launch_stage<2, RW, CW>(p2, g2, s);
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
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  WsHeader* hdr = (WsHeader*)ws;
  ColBlock* cbl = (ColBlock*)(ws + L.cbl);
  float* z = (float*)(ws + L.z);

  int RW, CW;
  if (a.T <= 16 && !a.multi) {
    RW = 1;
    CW = 1;
  } else if (a.T <= 64 && !a.multi) {
    RW = 2;
    CW = 2;
  } else {
    RW = 4;
    CW = 4;
  }
  if (a.multi) {
    const int64_t per = a.T / (a.num_adapters < a.T ? a.num_adapters : a.T);
    if (a.path == Path::Mfma && per <= 48) {
      RW = 2;
      CW = 2;
    }
  }
  const int chunk = 16 * CW;

  StageParams p{};
  p.T = a.T;
  p.ell = a.ell;
  p.x = a.x;
  p.ldx = a.ldx;
  p.z = z;
  p.ldz = ldz_of(a.R);
  p.zstride = a.T * p.ldz;
  p.y = a.y;
  p.ldy = a.ldy;
  p.y_f32 = a.y_f32;
  p.accumulate = a.accumulate;
  p.single = a.single;
  p.multi = a.multi;
  p.cbl = cbl;
  p.hdr = hdr;
  p.num_adapters = a.num_adapters;
  p.B1s = a.B1s;
  p.B2s = a.B2s;
  p.alphas = a.alphas;
  p.betas = a.betas;
  p.gammas = a.gammas;

  int64_t n_cb_max;
  if (a.multi) {
    hipError_t e = launch_segment(a, chunk, s);
    if (e != hipSuccess) return e;
    n_cb_max = a.T + cdiv(a.T, chunk);
    if (n_cb_max > max_colblocks(a.T)) n_cb_max = max_colblocks(a.T);
  } else {
    n_cb_max = cdiv(a.T, chunk);
    p.n_cb_host = n_cb_max;
  }

  StageParams p1 = p, p2 = p;
  p1.rows = a.R;
  p1.K = a.M;
  p1.nrt = cdiv(a.R, kRowTile);
  p1.nkb = cdiv(a.M, kColBlock);
  p2.rows = a.N;
  p2.K = a.R;
  p2.nrt = cdiv(a.N, kRowTile);
  p2.nkb = cdiv(a.R, kColBlock);

  if (RW == 1) return run_stages<1, 1>(p1, p2, a.multi, n_cb_max, s);
  if (RW == 2) return run_stages<2, 2>(p1, p2, a.multi, n_cb_max, s);
  return run_stages<4, 4>(p1, p2, a.multi, n_cb_max, s);
}

}  // namespace dbf
