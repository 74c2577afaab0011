// Large-T (prefill) path: the two sign-accumulation stages as fp16 matrix-
// core contractions.
//
// Once the signs are expanded to +-1 each stage is a dense contraction over
// the batch (DBF summary, section 2, inference: the product with the weight
// becomes two products with sign matrices), so it runs on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation; the operands gamma_i*x and
// z_i = beta_i*u_i are rounded to fp16.
//
// K order: the packed word a lane of group g holds for (row rho, 128-block)
// supplies the A operand of four 32-K steps s = 0..3, slots 8s..8s+7 each
// (bits s, s+4, ..., s+28), which are the block cols 32s + 8g + e, e = 0..7.
// The activation operand of lane group g, element e, step s is that same col,
// so both operands see the same k and no lane exchange is needed; one load
// instruction of step s reads 64 contiguous bytes (cols 32s..32s+31) of each
// of its 16 token rows.
//
// Work item: a column block of 16*NC tokens and either one row quad (64
// rows) whose reduction the four waves split (SPLITK: interleaved 128-blocks,
// partial tiles summed in a fixed order through LDS), or four row quads, one
// per wave, each over the whole reduction (for short reductions).  Output
// column j of an MFMA depends only on operand column j, so columns of tokens
// past the block's end read a valid token's row and are simply not stored.
// Stage 1 writes z_i = beta_i * u_i as fp16 into the workspace, in the order
// stage 2's MFMA operands take it (so each of its operand loads is 1 KB
// contiguous); stage 2 writes y = sum_i alpha_i * (B1 z_i).
#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

namespace {

typedef const DBF_GLOBAL v8h* gv8hp;

struct GemmParams {
  int32_t rows, K, T, nq, nkb, ell;
  int32_t n_cb_host, n_rg;  // column blocks (single adapter), row groups
  int32_t y_f32, accumulate, multi, xcd_remap;
  uint32_t msk16, one16;  // 0x80008000, 0x3C003C00 (kept in registers)
  const half_t* x;
  int64_t ldx;
  half_t* zt;         // z_i, fp16 in MFMA operand order (see zt_term_halfs)
  int64_t zt_term;    // halfs per term
  int32_t zt_nkb;     // 128-row blocks of z
  void* y;
  int64_t ldy;
  Factors single;
  const ColBlock* cbl;
  const WsHeader* hdr;
  const uint32_t* const* B1s;
  const uint32_t* const* B2s;
  const half_t* const* alphas;
  const half_t* const* betas;
  const half_t* const* gammas;
};

// A operand of step s for one lane: slots 8s..8s+7 of its word as fp16 +-1.
// Slot 8s+e sits at bit 4e+s, so halves (2p, 2p+1) come from bits 8p+s and
// 8p+4+s.  U = w << (7-s) puts bit 8p+s at bit 7 of byte p and V = w << (3-s)
// puts bit 8p+4+s there; a byte permute moves those bytes to bytes 1 and 3,
// and one and-or keeps bits 15 and 31 (msk = 0x80008000) and supplies the
// magnitude 1.0 (one = 0x3C003C00).
template <int s>
__device__ inline v8h expand_step_f16(uint32_t w, uint32_t msk, uint32_t one) {
  const uint32_t U = w << (7 - s), V = w << (3 - s);
  v4u o;
  o[0] = and_or(__builtin_amdgcn_perm(V, U, 0x040C000Cu), msk, one);
  o[1] = and_or(__builtin_amdgcn_perm(V, U, 0x050C010Cu), msk, one);
  o[2] = and_or(__builtin_amdgcn_perm(V, U, 0x060C020Cu), msk, one);
  o[3] = and_or(__builtin_amdgcn_perm(V, U, 0x070C030Cu), msk, one);
  return __builtin_bit_cast(v8h, o);
}

// Operands of one 128-block as loaded: sign words of the four row tiles,
// raw activations b[s][c] (k = kb*128 + 32s + 8g .. +7 of token column c)
// and, in stage 1, gamma over the same k.
template <int STAGE, int NC>
struct Block {
  v4u a;
  v8h b[4][NC];
  v8h gm[4];
};

// arow[c]: stage 1, the row of x of token column c (plus 8g); stage 2, the
// lane's 16 bytes of that token's z tile row, so step s of block kb sits at
// arow[c] + kb*2048 + s*512.
template <int STAGE, int NC>
__device__ inline const half_t* act_ptr(const half_t* arow, int kb, int s) {
  return STAGE == 1 ? arow + kb * kColBlock + 32 * s : arow + (int64_t)kb * 2048 + s * 512;
}

template <int STAGE, int NC>
__device__ inline void load_full(Block<STAGE, NC>& B, const char* sq, const half_t* const (&arow)[NC],
                                 int kb, int g) {
  B.a = *(gv4up)(sq + ((int64_t)kb << 10));
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int c = 0; c < NC; ++c) B.b[s][c] = *(gv8hp)act_ptr<STAGE, NC>(arow[c], kb, s);
}

// gamma of block kb from the LDS window that starts at block wb0
template <int STAGE, int NC>
__device__ inline void load_gamma(Block<STAGE, NC>& B, const half_t* gl, int kb, int wb0, int g) {
  if (STAGE == 1) {
    const v8h* gp = (const v8h*)(gl + (kb - wb0) * kColBlock + 8 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) B.gm[s] = gp[4 * s];
  }
}

// The last, partial 128-block: activations past K are zero (the padding
// signs are +1, so they must not contribute).  Cold code: not unrolled.
template <int STAGE, int NC>
__device__ inline void load_tail(Block<STAGE, NC>& B, const char* sq, const half_t* const (&arow)[NC],
                                 const half_t* gam, int kb, int g, int K) {
  B.a = *(gv4up)(sq + ((int64_t)kb << 10));
  const int kbase = kb * kColBlock + 8 * g;
  for (int s = 0; s < 4; ++s) {
    v8h gv = {};
    for (int e = 0; e < 8; ++e) {
      const int k = kbase + 32 * s + e;
      if (STAGE == 1 && k < K) gv[e] = gam[k];
    }
    B.gm[s] = gv;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      v8h v = {};
      if (STAGE == 1) {
        for (int e = 0; e < 8; ++e) {
          const int k = kbase + 32 * s + e;
          if (k < K) v[e] = arow[c][k - 8 * g];  // arow already points 8g in
        }
      } else if (kbase + 32 * s < K) {
        // the z tile spans the whole block; rows past K are not written
        v = *(gv8hp)act_ptr<STAGE, NC>(arow[c], kb, s);
        for (int e = 0; e < 8; ++e)
          if (kbase + 32 * s + e >= K) v[e] = (half_t)0.0f;
      }
      B.b[s][c] = v;
    }
  }
}

template <int STAGE, int NC>
__device__ inline void mma_block(v4f (&acc)[4][NC], const Block<STAGE, NC>& B, uint32_t msk,
                                 uint32_t one) {
  auto step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    v8h a[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) a[h] = expand_step_f16<s>(B.a[h], msk, one);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const v8h bv = STAGE == 1 ? B.b[s][c] * B.gm[s] : B.b[s][c];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        acc[h][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[h], bv, acc[h][c], 0, 0, 0);
    }
  };
  step(std::integral_constant<int, 0>{});
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 3>{});
}

// Blocks of gamma held in LDS at a time (a window of the reduction).
constexpr int kGamWindow = 128;

template <int STAGE, int NC, bool SPLITK>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  constexpr int D = 2;  // operand buffers per wave (deeper rings measured slower)
  __shared__ v4f red[SPLITK ? 4 : 1][SPLITK ? 4 * NC : 1][64];
  extern __shared__ v8h gam_lds[];  // stage 1: gamma_i over one window
  half_t* gl = (half_t*)gam_lds;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const uint32_t one = p.one16;
  const int n_cb = p.multi ? p.hdr->n_colblocks : p.n_cb_host;
  const int64_t n_items = (int64_t)n_cb * p.n_rg;
  // consecutive items share a column block; with the remap the items of one
  // XCD (workgroups b, b+8, ...) are consecutive, so they share activations
  // in that XCD's L2
  int64_t first = blockIdx.x;
  if (p.xcd_remap) first = (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int nfull = p.K / kColBlock;
  const bool has_tail = nfull < p.nkb;
  // stage 2 reads no gamma: one window spans the whole reduction
  const int win = STAGE == 1 ? kGamWindow : (nfull > 0 ? nfull : 1);

  for (int64_t it = first; it < n_items; it += gridDim.x) {
    const int cb = (int)(it / p.n_rg), rg = (int)(it % p.n_rg);
    int t0, t1, ad;
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
        f.gamma = p.gammas[ad];
      }
    } else {
      t0 = cb * 16 * NC;
      t1 = t0 + 16 * NC < p.T ? t0 + 16 * NC : p.T;
      ad = 0;
      f = p.single;
    }
    const int q = SPLITK ? rg : 4 * rg + wv;  // row quad of this wave
    const int row_lo = (SPLITK ? rg : 4 * rg) * kQuad * kRowTile;
    const int row_hi = min(p.rows, row_lo + (SPLITK ? 1 : 4) * kQuad * kRowTile);
    if (ad < 0) {
      // tokens whose adapter id is out of range: y = 0 (or unchanged)
      if (STAGE == 2 && !p.accumulate) {
        const int nr = row_hi - row_lo;
        for (int e = threadIdx.x; e < (t1 - t0) * nr; e += blockDim.x) {
          const int64_t t = t0 + e / nr, r = row_lo + e % nr;
          if (p.y_f32)
            ((float*)p.y)[t * p.ldy + r] = 0.0f;
          else
            ((half_t*)p.y)[t * p.ldy + r] = (half_t)0.0f;
        }
      }
      continue;
    }
    const bool active = SPLITK || q < p.nq;  // idle waves still reach every barrier
    const char* sq =
        (const char*)(STAGE == 1 ? f.B2 : f.B1) + ((int64_t)(active ? q : 0) * p.nkb << 10) + lane * 16;
    float ys[SPLITK ? NC : 4 * NC][4];  // stage 2: running sum over the terms

    for (int i = 0; i < p.ell; ++i) {
      // row scales of this wave's quad (lane L: row 64q + L), issued first so
      // that their latency hides behind the reduction; lanes fetch the ones
      // they need with a cross-lane read at the end
      // (kept as loaded; converting here would wait for the load)
      const half_t* sv = (STAGE == 1 ? f.beta : f.alpha) + (int64_t)i * p.rows;
      const int srow = q * kQuad * kRowTile + lane;
      const half_t sclh = sv[min(srow, p.rows - 1)];
      const half_t* arow[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int t = min(t0 + 16 * c + c16, t1 - 1);
        arow[c] = STAGE == 1 ? p.x + (int64_t)t * p.ldx + 8 * g
                             : p.zt + i * p.zt_term + (int64_t)(t >> 4) * p.zt_nkb * 2048 +
                                   (16 * g + (t & 15)) * 8;
      }
      const half_t* gam = STAGE == 1 ? f.gamma + (int64_t)i * p.K : nullptr;

      v4f acc[4][NC];
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[h][c] = v4f{0.f, 0.f, 0.f, 0.f};

      for (int wb0 = 0; wb0 < nfull; wb0 += win) {
        const int wb1 = min(nfull, wb0 + win);
        // this wave's blocks of the window: wb0+wv, wb0+wv+4, ... (SPLITK)
        // or all of them
        const int kb0 = wb0 + (SPLITK ? wv : 0), kst = SPLITK ? 4 : 1;
        const int nkw = SPLITK ? (wb1 - wb0 - wv + 3) / 4 : wb1 - wb0;
        const bool run = active && nkw > 0;
        // Operands of the next D-1 blocks are in flight while one is
        // consumed: D buffers with fixed roles (the loop is unrolled by D),
        // refilled right after their last use.  Every step issues the same
        // loads (clamped at the end), so each in-order wait covers exactly
        // the buffer about to be used.  The first D blocks are requested
        // before gamma is staged, so one memory round trip covers both.
        auto kb_of = [&](int j) {  // block of the wave's j-th step (clamped)
          return kb0 + min(j, nkw - 1) * kst;
        };
        Block<STAGE, NC> buf[D];
        if (run) {
#pragma unroll
          for (int d = 0; d < D; ++d) load_full<STAGE, NC>(buf[d], sq, arow, kb_of(d), g);
        }
        if (STAGE == 1) {
          // gamma of this window into LDS, element by element (any
          // alignment), eight loads in flight per thread
          __syncthreads();
          const int nk = (wb1 - wb0) * kColBlock;
          const half_t* gw = gam + wb0 * kColBlock;
          for (int k0 = 0; k0 < nk; k0 += 8 * 256) {
            half_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int k = k0 + e * 256 + threadIdx.x;
              v[e] = k < nk ? gw[k] : (half_t)0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int k = k0 + e * 256 + threadIdx.x;
              if (k < nk) gl[k] = v[e];
            }
          }
          __syncthreads();
        }
        if (!run) continue;
#pragma unroll
        for (int d = 0; d < D; ++d) load_gamma<STAGE, NC>(buf[d], gl, kb_of(d), wb0, g);
        for (int j = 0; j < nkw; j += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            if (j + d < nkw) mma_block<STAGE, NC>(acc, buf[d], p.msk16, one);
            __builtin_amdgcn_sched_barrier(0);
            const int kr = kb_of(j + d + D);
            load_full<STAGE, NC>(buf[d], sq, arow, kr, g);
            load_gamma<STAGE, NC>(buf[d], gl, kr, wb0, g);
          }
        }
      }
      if (has_tail && active && (!SPLITK || (nfull & 3) == wv)) {
        Block<STAGE, NC> bt;
        load_tail<STAGE, NC>(bt, sq, arow, gam, nfull, g, p.K);
        mma_block<STAGE, NC>(acc, bt, p.msk16, one);
      }

      if (SPLITK) {
        // fixed-order sum of the four waves' partial tiles; wave w finishes
        // tiles w*NC .. w*NC + NC-1 (tile = h*NC + c)
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int c = 0; c < NC; ++c) red[wv][h * NC + c][lane] = acc[h][c];
        __syncthreads();
      }
      if (active) {
        constexpr int NE = SPLITK ? NC : 4 * NC;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int tile = SPLITK ? wv * NC + e : e, h = tile / NC, c = tile % NC;
          v4f sum;
          if (SPLITK) {
            sum = ((red[0][tile][lane] + red[1][tile][lane]) + red[2][tile][lane]) +
                  red[3][tile][lane];
          } else {
            sum = acc[h][c];
          }
          const int rl = h * kRowTile + 4 * g;  // quad-local row of v = 0
          const int r0 = q * kQuad * kRowTile + rl;
          const int t = t0 + 16 * c + c16;
          const float scl = srow < p.rows ? (float)sclh : 0.0f;
          float sc[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[v] = __shfl(scl, rl + v, 64);
          if (STAGE == 1) {
            // rows r0..r0+3 share one 8-element chunk of the z tile; rows
            // past R get scale 0, so the chunk is written whole
            if (t < t1) {
              const int k = r0 & 127;
              half_t* zp = p.zt + i * p.zt_term +
                           ((int64_t)(t >> 4) * p.zt_nkb + (r0 >> 7)) * 2048 + (k >> 5) * 512 +
                           (16 * ((k >> 3) & 3) + (t & 15)) * 8 + (k & 7);
              *(v4h*)zp = v4h{(half_t)(sum[0] * sc[0]), (half_t)(sum[1] * sc[1]),
                              (half_t)(sum[2] * sc[2]), (half_t)(sum[3] * sc[3])};
            }
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float term = sum[v] * sc[v];
              ys[e][v] = (i == 0) ? term : ys[e][v] + term;
            }
            if (i + 1 == p.ell && t < t1 && r0 < p.rows) {
              float o[4] = {ys[e][0], ys[e][1], ys[e][2], ys[e][3]};
              if (p.accumulate) {
                float old[4];
                load4(p.y, p.ldy, p.y_f32, t, r0, p.rows, old);
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] += old[v];
              }
              store4(p.y, p.ldy, p.y_f32, t, r0, p.rows, o);
            }
          }
        }
      }
      if (SPLITK) __syncthreads();
    }
  }
}

template <int STAGE, int NC, bool SPLITK>
hipError_t launch_one(GemmParams p, hipStream_t s) {
  p.n_rg = SPLITK ? p.nq : (p.nq + 3) / 4;
  const int64_t items = (int64_t)p.n_cb_host * p.n_rg;
  int64_t grid = items;
  if (p.multi && grid > 8192) grid = 8192;
  p.xcd_remap = (grid == items && items % 8 == 0) ? 1 : 0;
  const int nfull = p.K / kColBlock;
  const size_t lds = STAGE == 1 ? (size_t)(nfull < kGamWindow ? nfull : kGamWindow) * kColBlock * 2 : 0;
  hipLaunchKernelGGL((k_gemm<STAGE, NC, SPLITK>), dim3((unsigned)grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

// Tokens per column block: 64 feeds each expanded sign operand to more
// MFMAs, 32 doubles the number of work items when 64 would leave compute
// units idle; the row-split variant (short reductions) always takes 32.
template <int STAGE>
hipError_t launch_stage(GemmParams p, hipStream_t s) {
  const bool split = p.nkb >= 4;
  if (p.multi) {
    return split ? launch_one<STAGE, 2, true>(p, s) : launch_one<STAGE, 2, false>(p, s);
  }
  if (split && cdiv(p.T, 64) * p.nq >= 512) {
    p.n_cb_host = (int32_t)cdiv(p.T, 64);
    return launch_one<STAGE, 4, true>(p, s);
  }
  p.n_cb_host = (int32_t)cdiv(p.T, 32);
  return split ? launch_one<STAGE, 2, true>(p, s) : launch_one<STAGE, 2, false>(p, s);
}

}  // namespace

hipError_t launch_gemm(const ForwardArgs& a, hipStream_t s) {
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  GemmParams p{};
  if (a.multi) {
    // column blocks of at most kGemmChunk tokens of one adapter
    if (a.stages & 1) {
      const hipError_t e = launch_segment(a, kGemmChunk, s);
      if (e != hipSuccess) return e;
    }
    int64_t n_cb = a.T + cdiv(a.T, kGemmChunk);
    if (n_cb > max_colblocks(a.T)) n_cb = max_colblocks(a.T);
    p.n_cb_host = (int32_t)n_cb;
  }
  p.T = (int32_t)a.T;
  p.ell = a.ell;
  p.msk16 = 0x80008000u;
  p.one16 = 0x3C003C00u;
  p.y_f32 = a.y_f32;
  p.accumulate = a.accumulate;
  p.multi = a.multi;
  p.x = a.x;
  p.ldx = a.ldx;
  p.zt = (half_t*)(ws + L.z);
  p.zt_term = zt_term_halfs(a.R, a.T);
  p.zt_nkb = (int32_t)cdiv(a.R, kColBlock);
  p.y = a.y;
  p.ldy = a.ldy;
  p.single = a.single;
  p.cbl = (const ColBlock*)(ws + L.cbl);
  p.hdr = (const WsHeader*)ws;
  p.B1s = a.B1s;
  p.B2s = a.B2s;
  p.alphas = a.alphas;
  p.betas = a.betas;
  p.gammas = a.gammas;

  GemmParams p1 = p, p2 = p;
  p1.rows = (int32_t)a.R;
  p1.K = (int32_t)a.M;
  p1.nq = (int32_t)cdiv(a.R, kRowTile * kQuad);
  p1.nkb = (int32_t)cdiv(a.M, kColBlock);
  p2.rows = (int32_t)a.N;
  p2.K = (int32_t)a.R;
  p2.nq = (int32_t)cdiv(a.N, kRowTile * kQuad);
  p2.nkb = (int32_t)cdiv(a.R, kColBlock);
  if (a.stages & 1) {
    const hipError_t e = launch_stage<1>(p1, s);
    if (e != hipSuccess) return e;
  }
  return (a.stages & 2) ? launch_stage<2>(p2, s) : hipSuccess;
}

}  // namespace dbf
