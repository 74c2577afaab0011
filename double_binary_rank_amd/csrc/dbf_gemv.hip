// Small-T (decode) path: the two sign-accumulation stages on the gfx950
// scaled fp4 x fp8 matrix core.
//
// The pages' kernel replaces the floating-point multiplies of the inner
// product by additions and subtractions of activations (LoRDBA summary,
// section 2 "Nucleo de Inferencia"; DBF summary, section 2 "Calculo en la
// inferencia").  Here a packed word of 32 signs becomes the fp4 (e2m1) A
// operand +-1.0 with one shift and one AND-OR per 8 signs, and the matrix
// core does the signed accumulation: every product is +-activation, so the
// MFMA performs exactly the adds and subtracts of the method.
//
// Activations are carried as three fp8 (e4m3) parts with a power-of-two
// scale per 128 values (E8M0, applied by the MFMA): part 0 rounds v, part 1
// rounds the remainder, part 2 the remainder of that.  The three parts hold
// about 12 significant bits of each value (integers up to 2^12 exactly) and
// occupy three of the 16 MFMA columns; their sums are added in fp32 in the
// epilogue.  So one 16x16x128 MFMA covers 16 rows x 128 reduction entries
// for up to floor(16 / (3*ell)) tokens x ell terms.
//
// Launches: prep(x) -> stage 1 (writes z = beta*u, fp32) -> prep(z) -> stage 2.
#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

// ------------------------------------------------------------ fp8 parts ----

__device__ inline int floor_log2_pos(float m) {
  return (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127;
}

// Round a (|a| < 256) to OCP e4m3 (3 mantissa bits, subnormal step 2^-9),
// nearest-even.  Returns the code; q receives the rounded value.  The code
// of a binade carry (mantissa 8 -> next exponent) follows from the encoding
// being monotonic in the magnitude.
__device__ inline uint32_t e4m3_rne(float a, float& q) {
  const uint32_t sgn = (__float_as_uint(a) >> 31) << 7;
  const float m = fabsf(a);
  const int e = floor_log2_pos(m);
  if (e < -6) {  // zero and the subnormal range
    const float qn = __builtin_rintf(m * 512.0f);  // 0..8; 8 encodes 2^-6 (0x08)
    q = __builtin_copysignf(qn * (1.0f / 512.0f), a);
    return sgn | (uint32_t)qn;
  }
  const float step = __builtin_ldexpf(1.0f, e - 3);
  const float qn = __builtin_rintf(m / step);  // 8..16
  q = __builtin_copysignf(qn * step, a);
  return sgn | (((uint32_t)(e + 7) << 3) + (uint32_t)(qn - 8.0f));
}

struct PrepParams {
  int64_t K, T, nkb;
  int32_t ell;
  int32_t from_z;  // 0: v = gamma_i * x_t (stage 1); 1: v = z_i,t (stage 2)
  const half_t* x;
  int64_t ldx;
  const float* z;
  int64_t ldz, zstride;
  const half_t* gamma;
  int32_t multi;
  const int32_t* ids;
  int32_t num_adapters;
  const half_t* const* gammas;
  uint32_t* opnd;  // [ell][T][nkb][kParts][4] x 8 words
  uint8_t* oscl;   // [ell][T][nkb][kParts][4]
};

// K order of an fp8 operand of v_mfma_scale_f32_16x16x128_f8f6f4 inside a
// 128-block: lane group g holds bytes e = 0..15 for k = 16g + e and bytes
// e = 16..31 for k = 64 + 16g + (e - 16).  (The fp4 operand holds 32
// consecutive k = 32g + e; measured on gfx950 with one-hot operands.)
__device__ inline int fp8_operand_k(int g, int e) { return e < 16 ? 16 * g + e : 48 + 16 * g + e; }

// One thread per (term, token, 128-block, lane group g); the four threads of
// a block are adjacent lanes.  Each loads the 32 values its lane group holds
// in the fp8 operand order, then the block is split into kParts fp8 parts.
// All four lane groups of a block share one E8M0 scale per part (the block
// maximum is exchanged with two lane shuffles), so the scale covers the
// whole 128-block whichever 32 of them the hardware attaches it to.
__global__ __launch_bounds__(256) void k_prep(PrepParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.ell * p.T * p.nkb * 4;
  const bool in = gid < total;  // out-of-range lanes still take part in the shuffles
  const int64_t gq = in ? gid : total - 1;
  const int g = (int)(gq & 3);
  int64_t rest = gq >> 2;
  const int64_t kb = rest % p.nkb;
  rest /= p.nkb;
  const int64_t t = rest % p.T;
  const int64_t i = rest / p.T;
  const int64_t kbase = kb * kColBlock;

  bool live = true;
  const half_t* gam = p.gamma;
  if (p.multi) {
    const int32_t ad = p.ids[t];
    live = ad >= 0 && ad < p.num_adapters;
    if (live && !p.from_z) gam = p.gammas[ad];
  }
  float v[32];
  if (!live) {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = 0.0f;
  } else if (p.from_z) {
    const float* zr = p.z + i * p.zstride + t * p.ldz;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int64_t k = kbase + fp8_operand_k(g, e);
      v[e] = k < p.K ? zr[k] : 0.0f;
    }
  } else {
    const half_t* gi = gam + i * p.K;
    const half_t* xr = p.x + t * p.ldx;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int64_t k = kbase + fp8_operand_k(g, e);
      v[e] = k < p.K ? (float)gi[k] * (float)xr[k] : 0.0f;
    }
  }

  const int64_t idx0 = ((i * p.T + t) * p.nkb + kb) * (kParts * 4);
#pragma unroll
  for (int part = 0; part < kParts; ++part) {
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(v[e]));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    int s = mx > 0.0f ? floor_log2_pos(mx) - 7 : 0;  // scaled block max in [128, 256)
    s = s < -127 ? -127 : (s > 127 ? 127 : s);
    const float down = __builtin_ldexpf(1.0f, -s), up = __builtin_ldexpf(1.0f, s);
    uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      float q;
      const uint32_t code = e4m3_rne(v[e] * down, q);
      v[e] -= q * up;  // exact: q*up is v rounded on a grid no finer than v's own
      words[e >> 2] |= code << (8 * (e & 3));
    }
    if (in) {
      const int64_t idx = idx0 + part * 4 + g;
      v4u* dst = (v4u*)(p.opnd + idx * 8);
      dst[0] = v4u{words[0], words[1], words[2], words[3]};
      dst[1] = v4u{words[4], words[5], words[6], words[7]};
      p.oscl[idx] = (uint8_t)(s + 127);
    }
  }
}

// ---------------------------------------------------------- stage kernel ----

// 32 sign slots of a packed word as fp4 (e2m1) +-1.0: register d holds slots
// 8d..8d+7, slot 8d+j in nibble j.  Slot 8d+j is stored at bit 4j+d, so a
// left shift by 3-d moves all eight sign bits to the nibble sign positions.
__device__ inline v8i expand_signs_fp4(uint32_t w) {
  v8i a;
  a[0] = (int)(((w << 3) & 0x88888888u) | 0x22222222u);
  a[1] = (int)(((w << 2) & 0x88888888u) | 0x22222222u);
  a[2] = (int)(((w << 1) & 0x88888888u) | 0x22222222u);
  a[3] = (int)((w & 0x88888888u) | 0x22222222u);
  a[4] = a[5] = a[6] = a[7] = 0;
  return a;
}

struct GemvParams {
  int64_t rows, K, T, nrt, nkb, n_rg;
  int32_t ell, tcb;
  const uint32_t* opnd;
  const uint8_t* oscl;
  float* z;
  int64_t ldz, zstride;
  void* y;
  int64_t ldy;
  int32_t y_f32, accumulate;
  Factors single;
  int32_t multi;
  const ColBlock* cbl;
  const WsHeader* hdr;
  int64_t n_cb_host;
  const uint32_t* const* B1s;
  const uint32_t* const* B2s;
  const half_t* const* alphas;
  const half_t* const* betas;
};

// Work item: (column block of <= tcb tokens, group of RTG row tiles).  The
// four waves split the reduction into interleaved chunks of KC blocks; each
// wave keeps the B operands of its chunk in registers and streams the sign
// blocks of all RTG row tiles against them.  Partial tiles are summed across
// waves in a fixed order through LDS.
template <int STAGE, int RTG>
__global__ __launch_bounds__(256) void k_gemv_fp4(GemvParams p) {
  constexpr int KC = 8;
  __shared__ v4f red[4][RTG][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int c = j / kParts, part = j - kParts * (j / kParts);
  const int64_t n_cb = p.multi ? (int64_t)p.hdr->n_colblocks : p.n_cb_host;
  const int64_t n_items = n_cb * p.n_rg;

  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t cb = it / p.n_rg, rg = it % p.n_rg;
    int64_t t0, t1;
    int32_t ad;
    Factors f;
    if (p.multi) {
      const ColBlock cbk = p.cbl[cb];
      t0 = cbk.t0;
      t1 = cbk.t1;
      ad = cbk.adapter;
      if (ad >= 0) {
        f.B1 = p.B1s[ad];
        f.B2 = p.B2s[ad];
        f.alpha = p.alphas[ad];
        f.beta = p.betas[ad];
      }
    } else {
      t0 = cb * p.tcb;
      t1 = t0 + p.tcb < p.T ? t0 + p.tcb : p.T;
      ad = 0;
      f = p.single;
    }
    const int64_t tile0 = rg * RTG;
    if (ad < 0) {
      if (STAGE == 2 && !p.accumulate) {
        const int64_t r0 = tile0 * kRowTile;
        const int64_t nr = (p.rows - r0) < RTG * kRowTile ? (p.rows - r0) : RTG * kRowTile;
        for (int64_t e = threadIdx.x; e < (t1 - t0) * nr; e += blockDim.x) {
          const int64_t t = t0 + e / nr, r = r0 + e % nr;
          if (p.y_f32)
            ((float*)p.y)[t * p.ldy + r] = 0.0f;
          else
            ((half_t*)p.y)[t * p.ldy + r] = (half_t)0.0f;
        }
      }
      continue;
    }
    const int ntok = (int)(t1 - t0);
    const int ncols = kParts * p.ell * ntok;
    const bool colv = j < ncols;
    const int ci = colv ? c / ntok : 0, ct = colv ? c - ntok * (c / ntok) : 0;
    const uint32_t* __restrict__ S = STAGE == 1 ? f.B2 : f.B1;

    v4f acc[RTG];
#pragma unroll
    for (int rt = 0; rt < RTG; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};

    const int64_t nrt_here = (p.nrt - tile0) < RTG ? (p.nrt - tile0) : RTG;
    for (int64_t kbase = 0; kbase < p.nkb; kbase += 4 * KC) {
      const int64_t kw0 = kbase + wv * KC;
      const int nk = (int)((p.nkb - kw0) < KC ? ((p.nkb - kw0) > 0 ? (p.nkb - kw0) : 0) : KC);
      if (nk == 0) continue;
      v8i bop[KC];
      int bsc[KC];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const int64_t kb = kw0 + kk;
        if (colv && kk < nk) {
          const int64_t idx = (((ci * p.T + t0 + ct) * p.nkb + kb) * kParts + part) * 4 + g;
          bop[kk] = *(gv8ip)(p.opnd + idx * 8);
          bsc[kk] = p.oscl[idx];
        } else {
          bop[kk] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          bsc[kk] = 127;
        }
      }
      gu32p base = (gu32p)S + (tile0 * p.nkb + kw0) * kBlockWords + lane;
      const int64_t tstride = p.nkb * kBlockWords;  // words between row tiles
      if (nk == KC && nrt_here == RTG) {
        // full chunk: two row tiles at a time, the next pair prefetched
        uint32_t wc[2][KC], wn[2][KC];
#pragma unroll
        for (int h = 0; h < 2 && h < RTG; ++h)
#pragma unroll
          for (int kk = 0; kk < KC; ++kk) wc[h][kk] = base[h * tstride + kk * kBlockWords];
#pragma unroll
        for (int rt = 0; rt < RTG; rt += 2) {
          if (rt + 2 < RTG) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int kk = 0; kk < KC; ++kk)
                wn[h][kk] = base[(rt + 2 + h) * tstride + kk * kBlockWords];
          }
#pragma unroll
          for (int kk = 0; kk < KC; ++kk)
#pragma unroll
            for (int h = 0; h < 2 && rt + h < RTG; ++h)
              acc[rt + h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  expand_signs_fp4(wc[h][kk]), bop[kk], acc[rt + h], 4 /* A: fp4 e2m1 */,
                  0 /* B: fp8 e4m3 */, 0, 127 /* A scale 2^0 */, 0, bsc[kk]);
          if (rt + 2 < RTG) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int kk = 0; kk < KC; ++kk) wc[h][kk] = wn[h][kk];
          }
        }
      } else {
        // ragged chunk or last row-tile group
#pragma unroll
        for (int rt = 0; rt < RTG; ++rt) {
          if (rt >= nrt_here) break;
          uint32_t w[KC];
#pragma unroll
          for (int kk = 0; kk < KC; ++kk)
            w[kk] = kk < nk ? base[rt * tstride + kk * kBlockWords] : 0u;
#pragma unroll
          for (int kk = 0; kk < KC; ++kk)
            acc[rt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                expand_signs_fp4(w[kk]), bop[kk], acc[rt], 4, 0, 0, 127, 0, bsc[kk]);
        }
      }
    }

#pragma unroll
    for (int rt = 0; rt < RTG; ++rt) red[wv][rt][lane] = acc[rt];
    __syncthreads();
    for (int rt = wv; rt < RTG; rt += 4) {
      const int64_t tile = tile0 + rt;
      if (tile >= p.nrt) break;
      const v4f sum = ((red[0][rt][lane] + red[1][rt][lane]) + red[2][rt][lane]) + red[3][rt][lane];
      const int64_t r0 = tile * kRowTile + 4 * g;
      float tot[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // parts of one column sit in lanes j, j+1, j+2 (same row group)
        const float d1 = __shfl(sum[v], lane + 1 < 64 ? lane + 1 : lane);
        const float d2 = __shfl(sum[v], lane + 2 < 64 ? lane + 2 : lane);
        tot[v] = (sum[v] + d1) + d2;
      }
      if (STAGE == 1) {
        if (part == 0 && colv && r0 < p.rows) {
          const half_t* bi = f.beta + (int64_t)ci * p.rows;
          float o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = (r0 + v < p.rows) ? tot[v] * (float)bi[r0 + v] : 0.0f;
          store4(p.z + ci * p.zstride, p.ldz, true, t0 + ct, r0, p.rows, o);
        }
      } else {
        const half_t* ai = f.alpha + (int64_t)ci * p.rows;
        float val[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          val[v] = (part == 0 && colv && r0 + v < p.rows) ? tot[v] * (float)ai[r0 + v] : 0.0f;
        // sum the ell terms of token ct: their part-0 lanes are 3*(i*ntok + ct)
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int ii = 0; ii < p.ell; ++ii) {
          int src = 16 * g + kParts * (ii * ntok + ct);
          src = src < 64 ? src : lane;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] += __shfl(val[v], src);
        }
        if (part == 0 && colv && ci == 0 && r0 < p.rows) {
          if (p.accumulate) {
            float old[4];
            load4(p.y, p.ldy, p.y_f32, t0 + ct, r0, p.rows, old);
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] += old[v];
          }
          store4(p.y, p.ldy, p.y_f32, t0 + ct, r0, p.rows, o);
        }
      }
    }
    __syncthreads();
  }
}

// -------------------------------------------------------------- launch ----

template <int STAGE, int RTG>
static hipError_t launch_gemv_stage(const GemvParams& p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_fp4<STAGE, RTG>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int STAGE>
static hipError_t launch_gemv_stage_any(GemvParams p, int64_t n_cb_est, int64_t n_cb_max,
                                        bool multi, hipStream_t s) {
  int rtg = 1;
  if (n_cb_est * cdiv(p.nrt, 16) >= 1024)
    rtg = 16;
  else if (n_cb_est * cdiv(p.nrt, 4) >= 1024)
    rtg = 4;
  p.n_rg = cdiv(p.nrt, rtg);
  int64_t grid = n_cb_max * p.n_rg;
  if (multi && grid > 4096) grid = 4096;
  if (rtg == 16) return launch_gemv_stage<STAGE, 16>(p, grid, s);
  if (rtg == 4) return launch_gemv_stage<STAGE, 4>(p, grid, s);
  return launch_gemv_stage<STAGE, 1>(p, grid, s);
}

static hipError_t launch_prep(PrepParams p, hipStream_t s) {
  const int64_t total = (int64_t)p.ell * p.T * p.nkb * 4;
  hipLaunchKernelGGL(k_prep, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv(const ForwardArgs& a, hipStream_t s) {
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  const int tcb = gemv_tokens_per_block(a.ell);
  hipError_t e;
  int64_t n_cb_max, n_cb_est;
  if (a.multi) {
    e = launch_segment(a, tcb, s);
    if (e != hipSuccess) return e;
    n_cb_max = a.T + cdiv(a.T, tcb);
    if (n_cb_max > max_colblocks(a.T)) n_cb_max = max_colblocks(a.T);
    n_cb_est = (int64_t)a.num_adapters + cdiv(a.T, tcb);
    if (n_cb_est > a.T) n_cb_est = a.T;
  } else {
    n_cb_max = n_cb_est = cdiv(a.T, tcb);
  }
  float* z = (float*)(ws + L.z);
  const int64_t ldz = ldz_of(a.R);

  PrepParams pp{};
  pp.T = a.T;
  pp.ell = a.ell;
  pp.x = a.x;
  pp.ldx = a.ldx;
  pp.z = z;
  pp.ldz = ldz;
  pp.zstride = a.T * ldz;
  pp.gamma = a.single.gamma;
  pp.multi = a.multi;
  pp.ids = a.ids;
  pp.num_adapters = a.num_adapters;
  pp.gammas = a.gammas;

  GemvParams gp{};
  gp.T = a.T;
  gp.ell = a.ell;
  gp.tcb = tcb;
  gp.z = z;
  gp.ldz = ldz;
  gp.zstride = a.T * ldz;
  gp.y = a.y;
  gp.ldy = a.ldy;
  gp.y_f32 = a.y_f32;
  gp.accumulate = a.accumulate;
  gp.single = a.single;
  gp.multi = a.multi;
  gp.cbl = (const ColBlock*)(ws + L.cbl);
  gp.hdr = (const WsHeader*)ws;
  gp.n_cb_host = n_cb_max;
  gp.B1s = a.B1s;
  gp.B2s = a.B2s;
  gp.alphas = a.alphas;
  gp.betas = a.betas;

  // stage 1: z = beta * (S2 . (gamma * x))
  pp.K = a.M;
  pp.nkb = cdiv(a.M, kColBlock);
  pp.from_z = 0;
  pp.opnd = (uint32_t*)(ws + L.p1o);
  pp.oscl = (uint8_t*)(ws + L.p1s);
  if ((e = launch_prep(pp, s)) != hipSuccess) return e;
  GemvParams g1 = gp;
  g1.rows = a.R;
  g1.K = a.M;
  g1.nrt = cdiv(a.R, kRowTile);
  g1.nkb = pp.nkb;
  g1.opnd = pp.opnd;
  g1.oscl = pp.oscl;
  if ((e = launch_gemv_stage_any<1>(g1, n_cb_est, n_cb_max, a.multi, s)) != hipSuccess) return e;

  // stage 2: y = sum_i alpha_i * (S1 . z_i)
  pp.K = a.R;
  pp.nkb = cdiv(a.R, kColBlock);
  pp.from_z = 1;
  pp.opnd = (uint32_t*)(ws + L.p2o);
  pp.oscl = (uint8_t*)(ws + L.p2s);
  if ((e = launch_prep(pp, s)) != hipSuccess) return e;
  GemvParams g2 = gp;
  g2.rows = a.N;
  g2.K = a.R;
  g2.nrt = cdiv(a.N, kRowTile);
  g2.nkb = pp.nkb;
  g2.opnd = pp.opnd;
  g2.oscl = pp.oscl;
  return launch_gemv_stage_any<2>(g2, n_cb_est, n_cb_max, a.multi, s);
}

}  // namespace dbf
