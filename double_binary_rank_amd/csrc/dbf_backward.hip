// Backward pass of one layer for quantisation-aware training (LoRDBA
// summary, section 2, "Pipeline de Entrenamiento", steps 3 and 4: sign
// carriers and scale vectors are trained together, the gradient passing
// sign() through a soft-sign straight-through estimator).
//
// With G = dL/dy [T][N] and, per term i, the forward's steps V_i = x.gamma_i,
// U_i = V_i S2^T, Z_i = U_i.beta_i, W_i = Z_i S1^T and the adjoint's steps
// P_i = (G.alpha_i) S1, Q_i = (P_i.beta_i) S2 (the chain rule on the update
// equation, "Arquitectura Central"):
//   dalpha_i = colsum(G . W_i),  dbeta_i = colsum(U_i . P_i),
//   dgamma_i = colsum(x . Q_i),  dx = sum_i Q_i . gamma_i,
//   dS1 = sum_i (G.alpha_i)^T Z_i,  dS2 = sum_i (P_i.beta_i)^T V_i,
//   dH = dS * (1 - tanh(H/tau)^2) / tau  (soft sign tanh(h/tau)).
//
// Launch sequence (one stream):
//   1. fp16 operand tiles of V_i and of G.alpha_i (k_prep_v2, one launch);
//   2. U_i = S2 V_i and P_i = S1^T (G.alpha_i): the large-T sign-product
//      kernel with raw fp32 output (k_gemm stage 3), P from the transposed
//      packing of S1;
//   3. tiles of Z_i = beta_i.U_i and of beta_i.P_i (k_tiles_f32);
//   4. W_i = S1 Z_i and Q_i = S2^T (beta_i.P_i), again stage 3;
//   5. the column dot products (coldot_block, colsum_block) and dx
//      (dx_block);
//   6. dS1, dS2 as dense fp16 matrix-core contractions over the tokens of
//      all terms (dense_block) from feature-major tiles (tiles_fm_block),
//      with the straight-through slope applied in the same epilogue.
// Independent work in one launch over task lists: the two k_tiles_f32; the
// three column dot products, dx and the four feature-major tiles
// (k_bwd_mid); the sums of the dot products' chunks and the two dense
// products (k_bwd_end); the two fp16 tile builds (k_prep_v2); with M = N
// the sign products two by two (grouped stage 3): 6 launches per call
// instead of 21 (8 with M != N).
// Every matrix-core operand is rounded to fp16 once from its exact fp32
// value, as on the forward large-T path; accumulation is fp32.
#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

namespace {

typedef const DBF_GLOBAL v8h* gv8hp;

// Up to kMaxTasks independent launches of one kernel as one launch: task j
// takes the workgroups [first[j], first[j + 1]).
constexpr int kMaxTasks = 4;
template <class P>
struct Tasks {
  P p[kMaxTasks];
  int64_t first[kMaxTasks + 1];
  int32_t n;
};

// The task of workgroup b (wave-uniform); b becomes the workgroup's index
// within its task.
template <class P>
__device__ inline const P& task_of(const Tasks<P>& t, int64_t& b) {
  int j = 0;
#pragma unroll
  for (int k = 1; k < kMaxTasks; ++k) j += (k < t.n && b >= t.first[k]) ? 1 : 0;
  b -= t.first[j];
  return t.p[j];
}

template <class P>
struct TaskList {
  Tasks<P> t{};
  void add(const P& p, int64_t blocks) {
    t.p[t.n] = p;
    t.first[t.n + 1] = t.first[t.n] + blocks;
    ++t.n;
  }
  int64_t blocks() const { return t.first[t.n]; }
};

// Token-major tiles (16 tokens x 128 reduction entries; entry (t, k) at
// half ((t/16 * nkb + k/128) * 4 + (k%128)/32) * 512 + (16 * (k/8 % 4) +
// t%16) * 8 + k%8 of its term) of fp16(scale_i[k] * src_i[t][k]), src fp32
// [ell][T][ld].  One thread per (term, token tile, 128-block, lane); it
// writes the lane's 8 entries of each of the 4 steps.
struct TilesF32Params {
  const float* src;
  int64_t ld, src_term;
  int32_t T, K, ell, nkb;
  int64_t n_units;
  const half_t* scale;  // [ell][K]
  half_t* out;
  int64_t out_term;
};

__global__ __launch_bounds__(256) void k_tiles_f32(Tasks<TilesF32Params> tasks) {
  int64_t b = blockIdx.x;
  const TilesF32Params& p = task_of(tasks, b);
  const int lane = threadIdx.x & 63;
  const int64_t u = b * 4 + (threadIdx.x >> 6);
  if (u >= p.n_units) return;
  const int kb = (int)(u % p.nkb);
  const int64_t r = u / p.nkb;
  const int ntt = (p.T + 15) >> 4;
  const int i = (int)(r / ntt), tt = (int)(r - (int64_t)i * ntt);
  const int g = lane >> 4, t = tt * 16 + (lane & 15);
  const float* row = p.src + i * p.src_term + (int64_t)t * p.ld;
  const half_t* sc = p.scale + (int64_t)i * p.K;
  half_t* out = p.out + i * p.out_term + ((int64_t)tt * p.nkb + kb) * 2048 + lane * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k0 = kb * kColBlock + 32 * s + 8 * g;
    v8h o = {};
    if (t < p.T)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + e < p.K) o[e] = (half_t)((float)sc[k0 + e] * row[k0 + e]);
    *(v8h*)(out + s * 512) = o;
  }
}

// Feature-major tiles for the sign gradients: the rows are the C features and
// the reduction runs over kappa = i * Tp + t (Tp = T rounded up to 128), each
// tile 16 features x 128 kappa in the same lane order, so a wave's 1 KB of a
// step is one MFMA operand.  Value fp16(scale_i[c] * src_i[t][c]); src is fp16
// [T][ld] shared by the terms (src16) or fp32 [ell][T][ld] (src32).  One
// thread per (feature tile, 128-block, step, lane): 8 tokens of one feature.
struct TilesFmParams {
  const half_t* src16;
  const float* src32;
  int64_t ld, src_term;
  int32_t T, C, Tp, nkb;  // nkb = ell * Tp / 128
  int64_t n_threads;
  const half_t* scale;  // [ell][C]
  half_t* out;
};

__device__ inline void tiles_fm_block(const TilesFmParams& p, int64_t b) {
  const int64_t id = b * blockDim.x + threadIdx.x;
  if (id >= p.n_threads) return;
  const int lane = (int)(id & 63), s = (int)((id >> 6) & 3);
  const int64_t blk = id >> 8;  // tile-major: (feature tile, 128-block)
  const int kb = (int)(blk % p.nkb);
  const int ct = (int)(blk / p.nkb);
  const int c = ct * 16 + (lane & 15);
  const int kappa = kb * kColBlock + 32 * s + 8 * (lane >> 4);
  const int i = kappa / p.Tp, t0 = kappa - i * p.Tp;
  v8h o = {};
  if (c < p.C) {
    const float sc = (float)p.scale[(int64_t)i * p.C + c];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t0 + e;
      if (t < p.T) {
        const float v = p.src16 != nullptr ? (float)p.src16[(int64_t)t * p.ld + c]
                                           : p.src32[i * p.src_term + (int64_t)t * p.ld + c];
        o[e] = (half_t)(sc * v);
      }
    }
  }
  *(v8h*)(p.out + blk * 2048 + s * 512 + lane * 8) = o;
}

// d_i[c] = sum_t a_i[t][c] * b_i[t][c] in fp32, deterministic: workgroup
// (column group of 64, token chunk of kColdotChunk) has 4 waves, wave w
// summing tokens w, w+4, ... of the chunk for 64 columns; the 4 partials are
// added in wave order and stored per chunk, and colsum_block adds the chunks in
// ascending order.  a is fp16 [T][lda] shared by the terms (a16) or fp32 per
// term (a32); b is fp32 [ell][T][ldb].
struct ColdotParams {
  const half_t* a16;
  const float* a32;
  int64_t lda, a_term;
  const float* b;
  int64_t ldb, b_term;
  int32_t T, C, ell, n_cg;  // n_cg: 64-column groups per term
  float* part;              // [chunks][ell][C]
  float* d;                 // [ell][C]
};

__device__ inline void coldot_block(const ColdotParams& p, int blk) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cg = blk % p.n_cg, i = (blk / p.n_cg) % p.ell;
  const int chunk = blk / (p.n_cg * p.ell);
  const int c = cg * 64 + lane;
  float acc = 0.0f;
  if (c < p.C) {
    const float* b = p.b + i * p.b_term + c;
    const int t1 = min(p.T, (chunk + 1) * kColdotChunk);
    if (p.a16 != nullptr) {
      const half_t* a = p.a16 + c;
      for (int t = chunk * kColdotChunk + wv; t < t1; t += 4)
        acc += (float)a[(int64_t)t * p.lda] * b[(int64_t)t * p.ldb];
    } else {
      const float* a = p.a32 + i * p.a_term + c;
      for (int t = chunk * kColdotChunk + wv; t < t1; t += 4)
        acc += a[(int64_t)t * p.lda] * b[(int64_t)t * p.ldb];
    }
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && c < p.C)
    p.part[((int64_t)chunk * p.ell + i) * p.C + c] =
        ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

struct ColsumParams {
  const float* part;  // [n_chunks][n]
  int32_t n_chunks;
  int64_t n;
  float* d;
};

__device__ inline void colsum_block(const ColsumParams& p, int64_t b) {
  const int64_t id = b * blockDim.x + threadIdx.x;
  if (id >= p.n) return;
  float acc = 0.0f;
  for (int k = 0; k < p.n_chunks; ++k) acc += p.part[(int64_t)k * p.n + id];
  p.d[id] = acc;
}

// dx[t][m] = sum_i gamma_i[m] * Q_i[t][m] (terms ascending), stored as fp16
// (nearest even) or fp32.
struct DxParams {
  const float* q;
  int64_t ldq, q_term;
  const half_t* gamma;
  int32_t T, M, ell;
  void* dx;
  int64_t lddx;
  int32_t f32;
};

__device__ inline void dx_block(const DxParams& p, int64_t b) {
  const int64_t id = b * blockDim.x + threadIdx.x;
  if (id >= (int64_t)p.T * p.M) return;
  const int64_t t = id / p.M, m = id - t * p.M;
  float acc = 0.0f;
  for (int i = 0; i < p.ell; ++i)
    acc += (float)p.gamma[(int64_t)i * p.M + m] * p.q[i * p.q_term + t * p.ldq + m];
  if (p.f32)
    ((float*)p.dx)[t * p.lddx + m] = acc;
  else
    ((half_t*)p.dx)[t * p.lddx + m] = (half_t)acc;
}

// Slope of the soft sign at y = h / tau, written as sech^2(y) =
// 4 e / (1 + e)^2 with e = exp(-2 |y|) (no cancellation for large |y|; e
// underflows to 0 there): one hardware exp2 and one reciprocal.
__device__ inline float sech2(float y) {
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * fabsf(y));  // -2 / ln 2
  const float d = 1.0f + e;
  return 4.0f * e * __builtin_amdgcn_rcpf(d * d);
}

// C[a][b] = sum_kappa A[a][kappa] * B[b][kappa] from feature-major tiles, on
// v_mfma_f32_16x16x32_f16.  A workgroup owns 128 A-rows x 128 B-rows, each
// of its 4 waves 64 x 64 (4 x 4 tiles) over the whole reduction; tiles past
// the matrices read as zero.  Epilogue: C (OUT) and the straight-through
// gradient C * sech^2(H * inv_tau) * inv_tau (STE).  A wave whose 64 x 64
// block lies inside both matrices stores without per-element checks.
struct DenseParams {
  const half_t* A;
  const half_t* B;
  int32_t nta, ntb, nkb;  // 16-row tiles of A and B, 128-blocks of the reduction
  int32_t rows_a, rows_b, n_ga;  // n_ga: 128-row groups of A
  float* out;
  const float* H;
  float inv_tau;
  float* dH;  // all three [rows_a][rows_b]
};

template <bool OUT, bool STE>
__device__ inline void dense_block(const DenseParams& p, int blk) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int ga = blk % p.n_ga, gb = blk / p.n_ga;
  const int ta0 = (ga * 2 + (wv & 1)) * 4, tb0 = (gb * 2 + (wv >> 1)) * 4;
  float* __restrict__ out = p.out;
  float* __restrict__ dH = p.dH;
  const float* __restrict__ Hm = p.H;
  const int64_t ldo = p.rows_b;
  // interior waves (all 16 tiles inside both matrices) request every H entry
  // they will scale before the products, so that its latency overlaps them,
  // and store through one row pointer per register, the 4 column tiles at
  // 64-byte immediate offsets
  const bool interior = (ta0 + 4) * 16 <= p.rows_a && (tb0 + 4) * 16 <= p.rows_b;
  float hv[4][4][4];  // [h][v][c]
  if (STE && interior) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t o = (int64_t)((ta0 + h) * 16 + 4 * g + v) * ldo + tb0 * 16 + c16;
#pragma unroll
        for (int c = 0; c < 4; ++c) hv[h][v][c] = Hm[o + 16 * c];
      }
  }
  v4f acc[4][4];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[h][c] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < p.nkb; ++kb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8h a[4], b[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int ta = ta0 + h, tb = tb0 + h;
        a[h] = ta < p.nta ? *(gv8hp)(p.A + ((int64_t)ta * p.nkb + kb) * 2048 + s * 512 + lane * 8)
                          : v8h{};
        b[h] = tb < p.ntb ? *(gv8hp)(p.B + ((int64_t)tb * p.nkb + kb) * 2048 + s * 512 + lane * 8)
                          : v8h{};
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[h][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[h], b[c], acc[h][c], 0, 0, 0);
    }
  }
  // lane (g, c16), register v of tile (h, c): row 4g + v of A-tile h, row c16
  // of B-tile c
  if (interior) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t o = (int64_t)((ta0 + h) * 16 + 4 * g + v) * ldo + tb0 * 16 + c16;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float val = acc[h][c][v];
          if (OUT) out[o + 16 * c] = val;
          if (STE) dH[o + 16 * c] = val * (sech2(hv[h][v][c] * p.inv_tau) * p.inv_tau);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int rb = (tb0 + c) * 16 + c16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ra = (ta0 + h) * 16 + 4 * g + v;
        if (ra < p.rows_a && rb < p.rows_b) {
          const int64_t o = (int64_t)ra * ldo + rb;
          const float val = acc[h][c][v];
          if (OUT) out[o] = val;
          if (STE) dH[o] = val * (sech2(Hm[o] * p.inv_tau) * p.inv_tau);
        }
      }
    }
}

// The launch after the sign products W and Q: the three column dot
// products (workgroups [0, cd_end)), dx ([cd_end, dx_end)) and the
// feature-major tiles of the sign gradients ([dx_end, ...)).  They read only
// what earlier launches wrote.
struct MidParams {
  Tasks<ColdotParams> cd;
  DxParams dx;
  Tasks<TilesFmParams> fm;
  int64_t cd_end, dx_end;
};

__global__ __launch_bounds__(256) void k_bwd_mid(MidParams m) {
  int64_t b = blockIdx.x;
  if (b < m.cd_end) {
    const ColdotParams& p = task_of(m.cd, b);
    coldot_block(p, (int)b);
  } else if (b < m.dx_end) {
    dx_block(m.dx, b - m.cd_end);
  } else {
    b -= m.dx_end;
    const TilesFmParams& p = task_of(m.fm, b);
    tiles_fm_block(p, b);
  }
}

// The last launch: the sums of the dot products' chunks (workgroups [0,
// cs_end)) and the sign-gradient products with one epilogue.
struct EndParams {
  Tasks<ColsumParams> cs;
  Tasks<DenseParams> dn;
  int64_t cs_end;
};

template <bool OUT, bool STE>
__global__ __launch_bounds__(256) void k_bwd_end(EndParams e) {
  int64_t b = blockIdx.x;
  if (b < e.cs_end) {
    const ColsumParams& p = task_of(e.cs, b);
    colsum_block(p, b);
  } else {
    b -= e.cs_end;
    const DenseParams& p = task_of(e.dn, b);
    dense_block<OUT, STE>(p, (int)b);
  }
}

TilesF32Params tiles_f32(const float* src, int64_t ld, int64_t src_term, int64_t T, int64_t K,
                         int32_t ell, const half_t* scale, half_t* out) {
  TilesF32Params p{};
  p.src = src;
  p.ld = ld;
  p.src_term = src_term;
  p.T = (int32_t)T;
  p.K = (int32_t)K;
  p.ell = ell;
  p.nkb = (int32_t)cdiv(K, kColBlock);
  p.n_units = (int64_t)ell * cdiv(T, 16) * p.nkb;
  p.scale = scale;
  p.out = out;
  p.out_term = zt_term_halfs(K, T);
  return p;
}

TilesFmParams tiles_fm(const half_t* src16, const float* src32, int64_t ld, int64_t src_term,
                       int64_t T, int64_t C, int32_t ell, const half_t* scale, half_t* out) {
  TilesFmParams p{};
  p.src16 = src16;
  p.src32 = src32;
  p.ld = ld;
  p.src_term = src_term;
  p.T = (int32_t)T;
  p.C = (int32_t)C;
  p.Tp = (int32_t)(cdiv(T, 128) * 128);
  p.nkb = (int32_t)(bwd_kf(ell, T) / 128);
  p.n_threads = cdiv(C, 16) * p.nkb * 256;
  p.scale = scale;
  p.out = out;
  return p;
}

DenseParams dense(const half_t* A, const half_t* B, int64_t rows_a, int64_t rows_b, int64_t kf,
                  float* out, const float* H, float tau, float* dH) {
  DenseParams p{};
  p.A = A;
  p.B = B;
  p.nta = (int32_t)cdiv(rows_a, 16);
  p.ntb = (int32_t)cdiv(rows_b, 16);
  p.nkb = (int32_t)(kf / 128);
  p.rows_a = (int32_t)rows_a;
  p.rows_b = (int32_t)rows_b;
  p.n_ga = (int32_t)cdiv(rows_a, 128);
  p.out = out;
  p.H = H;
  p.inv_tau = H != nullptr ? 1.0f / tau : 0.0f;
  p.dH = dH;
  return p;
}

int64_t dense_blocks(const DenseParams& p) { return (int64_t)p.n_ga * cdiv(p.rows_b, 128); }

template <class P>
bool grid_ok(const TaskList<P>& l) {
  return l.t.n > 0 && l.blocks() <= INT32_MAX;
}

// One k_bwd_end launch: the column sums in `cs` (may be empty) and the dense
// products in `dn` (may be empty), which share one epilogue: out and dH of
// the first select it.
hipError_t launch_end(const TaskList<ColsumParams>& cs, const TaskList<DenseParams>& dn,
                      hipStream_t s) {
  EndParams e{};
  e.cs = cs.t;
  e.dn = dn.t;
  e.cs_end = cs.blocks();
  const int64_t grid = cs.blocks() + dn.blocks();
  if (grid <= 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const bool out = dn.t.n == 0 || dn.t.p[0].out != nullptr;
  const bool ste = dn.t.n > 0 && dn.t.p[0].H != nullptr;
  const dim3 g((unsigned)grid), b(256);
  if (out && ste)
    hipLaunchKernelGGL((k_bwd_end<true, true>), g, b, 0, s, e);
  else if (out)
    hipLaunchKernelGGL((k_bwd_end<true, false>), g, b, 0, s, e);
  else
    hipLaunchKernelGGL((k_bwd_end<false, true>), g, b, 0, s, e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  const BwdLayout L = bwd_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  half_t* vt = (half_t*)(ws + L.vt);
  half_t* gt = (half_t*)(ws + L.gt);
  float* u = (float*)(ws + L.u);
  float* pp = (float*)(ws + L.p);
  half_t* zt = (half_t*)(ws + L.zt);
  half_t* pt = (half_t*)(ws + L.pt);
  float* w = (float*)(ws + L.w);
  float* q = (float*)(ws + L.q);
  const int64_t T = a.T, N = a.N, R = a.R, M = a.M;
  const int32_t ell = a.ell;
  hipError_t e;
#define DBF_TRY(x) \
  if ((e = (x)) != hipSuccess) return e
  const int64_t lr = bwd_ld(R), ln = bwd_ld(N), lm = bwd_ld(M);
  // 1-2: U_i = S2 (gamma_i x), P_i = S1^T (alpha_i G)
  DBF_TRY(launch_tiles_f16_pair(TilesF16{a.x, a.ldx, M, a.gamma, vt},
                                TilesF16{a.g, a.ldg, N, a.alpha, gt}, T, ell, s));
  // with M = N the two products have one shape: one grouped launch
  const bool square = M == N;
  if (square) {
    DBF_TRY(launch_sign_product_pair(a.B2, a.B1t, R, M, ell, T, vt, gt, u, pp, lr, s));
  } else {
    DBF_TRY(launch_sign_product(a.B2, R, M, ell, T, vt, u, lr, s));
    DBF_TRY(launch_sign_product(a.B1t, R, N, ell, T, gt, pp, lr, s));
  }
  // 3-4: W_i = S1 (beta_i U_i), Q_i = S2^T (beta_i P_i)
  {
    TaskList<TilesF32Params> l;
    for (const TilesF32Params& q : {tiles_f32(u, lr, T * lr, T, R, ell, a.beta, zt),
                                    tiles_f32(pp, lr, T * lr, T, R, ell, a.beta, pt)})
      l.add(q, cdiv(q.n_units, 4));
    if (!grid_ok(l)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_tiles_f32, dim3((unsigned)l.blocks()), dim3(256), 0, s, l.t);
    DBF_TRY(hipGetLastError());
  }
  if (square) {
    DBF_TRY(launch_sign_product_pair(a.B1, a.B2t, N, R, ell, T, zt, pt, w, q, ln, s));
  } else {
    DBF_TRY(launch_sign_product(a.B1, N, R, ell, T, zt, w, ln, s));
    DBF_TRY(launch_sign_product(a.B2t, M, R, ell, T, pt, q, lm, s));
  }
  // 5-6: the scale gradients, dx and the sign gradients in two launches: the
  // column dot products, dx and the feature-major tiles, then the sums of
  // the dot products' chunks and the dense sign-gradient products.  The
  // three dot products keep their per-chunk partial sums in separate thirds
  // of the part region.
  float* part = (float*)(ws + L.part);
  const int64_t n_chunks = cdiv(T, kColdotChunk);
  const int64_t third = n_chunks * ell * bwd_colmax(N, R, M);
  const ColdotParams cd[3] = {
      {a.g, nullptr, a.ldg, 0, w, ln, T * ln, (int32_t)T, (int32_t)N, ell, (int32_t)cdiv(N, 64),
       part, a.dalpha},
      {nullptr, u, lr, T * lr, pp, lr, T * lr, (int32_t)T, (int32_t)R, ell, (int32_t)cdiv(R, 64),
       part + third, a.dbeta},
      {a.x, nullptr, a.ldx, 0, q, lm, T * lm, (int32_t)T, (int32_t)M, ell, (int32_t)cdiv(M, 64),
       part + 2 * third, a.dgamma}};
  TaskList<ColdotParams> lcd;
  TaskList<ColsumParams> lcs;
  for (const ColdotParams& c : cd) {
    lcd.add(c, (int64_t)c.n_cg * ell * n_chunks);
    const int64_t n = (int64_t)ell * c.C;
    lcs.add(ColsumParams{c.part, (int32_t)n_chunks, n, c.d}, cdiv(n, 256));
  }
  const int64_t kf = bwd_kf(ell, T);
  const bool want1 = a.dS1 != nullptr || a.dH1 != nullptr;
  const bool want2 = a.dS2 != nullptr || a.dH2 != nullptr;
  half_t* gf = (half_t*)(ws + L.gf);
  half_t* zf = (half_t*)(ws + L.zf);
  half_t* pf = (half_t*)(ws + L.pf);
  half_t* vf = (half_t*)(ws + L.vf);
  TaskList<TilesFmParams> lfm;
  {
    auto add = [&](const TilesFmParams& f) { lfm.add(f, cdiv(f.n_threads, 256)); };
    if (want1) {
      add(tiles_fm(a.g, nullptr, a.ldg, 0, T, N, ell, a.alpha, gf));
      add(tiles_fm(nullptr, u, lr, T * lr, T, R, ell, a.beta, zf));
    }
    if (want2) {
      add(tiles_fm(nullptr, pp, lr, T * lr, T, R, ell, a.beta, pf));
      add(tiles_fm(a.x, nullptr, a.ldx, 0, T, M, ell, a.gamma, vf));
    }
  }
  {
    MidParams m{};
    m.cd = lcd.t;
    m.dx = DxParams{q, lm, T * lm, a.gamma, (int32_t)T, (int32_t)M, ell, a.dx, a.lddx,
                    a.dx_f32 ? 1 : 0};
    m.fm = lfm.t;
    m.cd_end = lcd.blocks();
    m.dx_end = m.cd_end + cdiv(T * M, 256);
    const int64_t grid = m.dx_end + lfm.blocks();
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_bwd_mid, dim3((unsigned)grid), dim3(256), 0, s, m);
    DBF_TRY(hipGetLastError());
  }
  const DenseParams d1 = dense(gf, zf, N, R, kf, a.dS1, a.H1, a.tau, a.dH1);
  const DenseParams d2 = dense(pf, vf, R, M, kf, a.dS2, a.H2, a.tau, a.dH2);
  // both products with the column sums when they take the same epilogue
  const bool same = want1 && want2 && (a.dS1 != nullptr) == (a.dS2 != nullptr) &&
                    (a.H1 != nullptr) == (a.H2 != nullptr);
  TaskList<DenseParams> ldn;
  if (want1) ldn.add(d1, dense_blocks(d1));
  if (want2 && (same || !want1)) ldn.add(d2, dense_blocks(d2));
  DBF_TRY(launch_end(lcs, ldn, s));
  if (want1 && want2 && !same) {
    TaskList<ColsumParams> none;
    TaskList<DenseParams> l2;
    l2.add(d2, dense_blocks(d2));
    DBF_TRY(launch_end(none, l2, s));
  }
#undef DBF_TRY
  return hipSuccess;
}

}  // namespace dbf
