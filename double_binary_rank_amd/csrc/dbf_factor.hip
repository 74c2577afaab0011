// DBF factorisation of a dense weight matrix (DBF summary, section 2,
// "Algoritmo de Optimizacion"): W (N x M) ~ X Y with X = diag(a) A diag(m)
// (N x k) and Y = diag(r) B diag(b) (k x M), A and B sign matrices, by
// alternating minimisation; each half step is an ADMM run (scaled form,
// penalty rho = rho0 * trace(Gram) / k) whose projection onto the scaled sign
// matrices is SVID: sign times the rank-1 approximation of the magnitude.
//
// Everything is fp32 on the device, one stream:
//   * products of dense matrices: k_sgemm (fp32 matrix-core tiles of
//     128 x 128 through LDS; NN, NT and TN operand orders);
//   * the k x k solve (Gram + rho I)^-1 by Newton-Schulz iteration,
//     X <- X (2I - A X) from X0 = I / ||A||_inf, a fixed count of
//     2 ceil(log2(k + 1)) + 10 steps (the initial error is below 1 - 1/cond and
//     cond <= k + 1 here, so the count reaches fp32 accuracy);
//   * the top singular pair of |T| by power iteration (k_absmv_rows,
//     k_absmv_cols + k_norm_cols), warm-started from the previous projection
//     of the same side;
//   * the ADMM updates as fused elementwise kernels.
// Scalars that steer the iteration (rho, the Newton-Schulz start, norms) stay
// in device memory, so the host launches the whole schedule without waiting.
#include <climits>

#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

namespace {

// ------------------------------------------------------------- SGEMM ----
// C[m][n] = sum_k A(m,k) B(k,n); A(m,k) = A[m*lda + k] (TA: A[k*lda + m]),
// B(k,n) = B[k*ldb + n] (TB: B[n*ldb + k]).  fp32 in, fp32 accumulate, on
// the matrix core (v_mfma_f32_16x16x4_f32: twice the unpacked vector FMA
// rate).  A workgroup of 4 waves owns an MT x MT tile of C (MT = 128 or
// 64), each wave an MT/2 x MT/2 quarter as 16 x 16 MFMA tiles.  kMK-deep
// slices of A and B go
// through LDS, rows padded by 16 floats so that the 4 rows x 16 columns a
// wave reads per operand hit 64 distinct banks; the next slice is read from
// memory into registers while the current one is multiplied.
// MFMA lane layout (16 x 16 x 4): lane l holds A(l % 16, l / 16) and
// B(l / 16, l % 16); output register r of lane l is C(4 (l / 16) + r, l % 16).
constexpr int kMK = 16;

template <bool TA, bool TB, int MT>
__global__ __launch_bounds__(256) void k_sgemm(const float* __restrict__ A, int64_t lda,
                                               const float* __restrict__ B, int64_t ldb,
                                               float* __restrict__ C, int64_t ldc, int32_t Mr,
                                               int32_t Nc, int32_t K) {
  constexpr int MP = MT + 16;          // padded LDS row
  constexpr int ME = MT * kMK / 256;   // entries of each operand per thread and slice
  constexpr int WT = MT / 2;           // wave tile (2 x 2 waves)
  constexpr int NI = WT / 16;          // MFMA tiles per wave and dimension
  __shared__ float As[kMK][MP];  // As[k][m]
  __shared__ float Bs[kMK][MP];  // Bs[k][n]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_tn = (Nc + MT - 1) / MT;
  const int m0 = (int)(blockIdx.x / n_tn) * MT, n0 = (int)(blockIdx.x % n_tn) * MT;
  const int wm = (wv >> 1) * WT, wn = (wv & 1) * WT;
  // entry e of this thread in a slice: consecutive threads take
  // consecutive addresses of the source
  auto a_pos = [&](int e, int& m, int& k) {
    const int id = tid + 256 * e;
    if (TA) { k = id / MT; m = id % MT; } else { m = id / kMK; k = id % kMK; }
  };
  auto b_pos = [&](int e, int& k, int& n) {
    const int id = tid + 256 * e;
    if (TB) { n = id / kMK; k = id % kMK; } else { k = id / MT; n = id % MT; }
  };
  float ra[ME], rb[ME];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int e = 0; e < ME; ++e) {
      int m, k, kb, n;
      a_pos(e, m, k);
      b_pos(e, kb, n);
      const int gm = m0 + m, gk = k0 + k, gn = n0 + n, gkb = k0 + kb;
      ra[e] = (gm < Mr && gk < K) ? (TA ? A[(int64_t)gk * lda + gm] : A[(int64_t)gm * lda + gk]) : 0.0f;
      rb[e] = (gn < Nc && gkb < K) ? (TB ? B[(int64_t)gn * ldb + gkb] : B[(int64_t)gkb * ldb + gn]) : 0.0f;
    }
  };
  v4f acc[NI][NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += kMK) {
    __syncthreads();  // the previous slice's readers are done
#pragma unroll
    for (int e = 0; e < ME; ++e) {
      int m, k, kb, n;
      a_pos(e, m, k);
      b_pos(e, kb, n);
      As[k][m] = ra[e];
      Bs[kb][n] = rb[e];
    }
    __syncthreads();
    if (k0 + kMK < K) fetch(k0 + kMK);
#pragma unroll
    for (int k4 = 0; k4 < kMK / 4; ++k4) {
      const int kk = 4 * k4 + (lane >> 4), c = lane & 15;
      float a[NI], b[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) a[i] = As[kk][wm + 16 * i + c];
#pragma unroll
      for (int j = 0; j < NI; ++j) b[j] = Bs[kk][wn + 16 * j + c];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int gn = n0 + wn + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gm = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
        if (gm < Mr && gn < Nc) C[(int64_t)gm * ldc + gn] = acc[i][j][r];
      }
    }
}

// 128 x 128 tiles (64 x 64 per wave) when they give at least two workgroups
// per compute unit; 64 x 64 tiles otherwise, so that a product of a few
// hundred large tiles still keeps several waves on every SIMD.
template <bool TA, bool TB>
hipError_t sgemm(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                 int64_t Mr, int64_t Nc, int64_t K, hipStream_t s) {
  const int64_t big = cdiv(Mr, 128) * cdiv(Nc, 128);
  const bool small = big < 2 * 256;
  const int64_t grid = small ? cdiv(Mr, 64) * cdiv(Nc, 64) : big;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (small)
    hipLaunchKernelGGL((k_sgemm<TA, TB, 64>), dim3((unsigned)grid), dim3(256), 0, s, A, lda, B, ldb,
                       C, ldc, (int32_t)Mr, (int32_t)Nc, (int32_t)K);
  else
    hipLaunchKernelGGL((k_sgemm<TA, TB, 128>), dim3((unsigned)grid), dim3(256), 0, s, A, lda, B,
                       ldb, C, ldc, (int32_t)Mr, (int32_t)Nc, (int32_t)K);
  return hipGetLastError();
}

// ------------------------------------------------------- small kernels ----
// Device scalars (floats at sc[]):
enum Scalar { kRho = 0, kNsC = 1, kNrm = 2, kErr = 3, kWn = 4, kNScalars = 8 };

// One workgroup of 1024 threads: sum of v[i * stride] for i < n, fixed order
// per thread, then a tree in LDS (deterministic).
__device__ inline float block_sum(float x) {
  __shared__ float red[1024];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// Absolute column sums of the k x k matrix G + rho I.  A workgroup of 16
// waves owns 64 columns (lane = column); wave w sums rows w, w + 16, ...,
// and the 16 partial sums are added in wave order.  rho comes from the
// trace summed exactly as k_regularise sums it.
__global__ __launch_bounds__(1024) void k_colabs(const float* G, int32_t k, float rho0, float* cs) {
  float tr = 0.0f;
  for (int i = threadIdx.x; i < k; i += 1024) tr += G[(int64_t)i * k + i];
  const float rho = rho0 * block_sum(tr) / (float)k;
  __shared__ float part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  float a = 0.0f;
  if (j < k) {
#pragma unroll 8
    for (int i = w; i < k; i += 16) a += fabsf(G[(int64_t)i * k + j] + (i == j ? rho : 0.0f));
  }
  part[w][lane] = a;
  __syncthreads();
  if (w == 0 && j < k) {
    float t = 0.0f;
    for (int v = 0; v < 16; ++v) t += part[v][lane];
    cs[j] = t;
  }
}

// rho = rho0 * trace(G) / k;  A = G + rho I (in place);  Newton-Schulz start
// constant 1 / ||A||_inf (A is symmetric: the largest absolute column sum,
// from cs).
__global__ __launch_bounds__(1024) void k_regularise(float* G, int32_t k, float rho0,
                                                     const float* cs, float* sc) {
  float tr = 0.0f;
  for (int i = threadIdx.x; i < k; i += 1024) tr += G[(int64_t)i * k + i];
  const float rho = rho0 * block_sum(tr) / (float)k;
  float mx = 0.0f;
  for (int j = threadIdx.x; j < k; j += 1024) mx = fmaxf(mx, cs[j]);
  __shared__ float mred[1024];
  mred[threadIdx.x] = mx;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) mred[threadIdx.x] = fmaxf(mred[threadIdx.x], mred[threadIdx.x + w]);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < k; i += 1024) G[(int64_t)i * k + i] += rho;
  if (threadIdx.x == 0) {
    sc[kRho] = rho;
    sc[kNsC] = 1.0f / mred[0];
  }
}

__global__ __launch_bounds__(256) void k_fill(float* v, int64_t n, float val) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < n) v[id] = val;
}

__global__ __launch_bounds__(256) void k_copy(float* dst, const float* src, int64_t n) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < n) dst[id] = src[id];
}

// X = c I (c from sc[kNsC])
__global__ __launch_bounds__(256) void k_ns_init(float* X, int32_t k, const float* sc) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)k * k) return;
  X[id] = (id / k == id % k) ? sc[kNsC] : 0.0f;
}

// T = 2I - T
__global__ __launch_bounds__(256) void k_two_minus(float* T, int32_t k) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)k * k) return;
  T[id] = (id / k == id % k ? 2.0f : 0.0f) - T[id];
}

// rhs = base + rho (Z - U)
__global__ __launch_bounds__(256) void k_rhs(const float* base, const float* Z, const float* U,
                                             float* rhs, int64_t n, const float* sc) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n) return;
  rhs[id] = base[id] + sc[kRho] * (Z[id] - U[id]);
}

// T = X + U (in X)
__global__ __launch_bounds__(256) void k_add(float* X, const float* U, int64_t n) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < n) X[id] += U[id];
}

// u[i] = sum_j |T[i][j]| v[j]: one wave per row.
__global__ __launch_bounds__(256) void k_absmv_rows(const float* T, int32_t rows, int32_t cols,
                                                    const float* v, float* u) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* t = T + (int64_t)row * cols;
  float acc = 0.0f;
  for (int j = lane; j < cols; j += 64) acc += fabsf(t[j]) * v[j];
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) u[row] = acc;
}

// Partial column sums part[chunk][j] = sum_{i in chunk} |T[i][j]| u[i] over
// chunks of 64 rows; 64 columns x 4 row groups per workgroup.
constexpr int kRowChunk = 64;
__global__ __launch_bounds__(256) void k_absmv_cols(const float* T, int32_t rows, int32_t cols,
                                                    const float* u, float* part) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n_cg = (cols + 63) / 64;
  const int cg = blockIdx.x % n_cg, chunk = blockIdx.x / n_cg;
  const int j = cg * 64 + lane;
  float acc = 0.0f;
  if (j < cols) {
    const int i1 = min(rows, (chunk + 1) * kRowChunk);
    for (int i = chunk * kRowChunk + wv; i < i1; i += 4) acc += fabsf(T[(int64_t)i * cols + j]) * u[i];
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && j < cols)
    part[(int64_t)chunk * cols + j] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// v[j] = sum_chunks part[c][j], then v /= ||v||_2 (one workgroup).
__global__ __launch_bounds__(1024) void k_norm_cols(const float* part, int32_t n_chunks,
                                                    int32_t cols, float* v) {
  float ss = 0.0f;
  for (int j = threadIdx.x; j < cols; j += 1024) {
    float a = 0.0f;
#pragma unroll 8
    for (int c = 0; c < n_chunks; ++c) a += part[(int64_t)c * cols + j];
    v[j] = a;
    ss += a * a;
  }
  const float nrm = sqrtf(block_sum(ss));
  const float inv = nrm > 0.0f ? 1.0f / nrm : 0.0f;
  __syncthreads();
  for (int j = threadIdx.x; j < cols; j += 1024) v[j] *= inv;
}

// After the last power step (v unit, u = |T| v = sigma * u_unit):
// s = ||u||; u <- u / sqrt(s), v <- v * sqrt(s) (the split of sigma).
__global__ __launch_bounds__(1024) void k_split(float* u, int32_t rows, float* v, int32_t cols) {
  float ss = 0.0f;
  for (int i = threadIdx.x; i < rows; i += 1024) ss += u[i] * u[i];
  const float sig = sqrtf(block_sum(ss));
  const float r = sqrtf(sig);
  const float iu = r > 0.0f ? 1.0f / r : 0.0f;
  __syncthreads();
  for (int i = threadIdx.x; i < rows; i += 1024) u[i] *= iu;
  for (int j = threadIdx.x; j < cols; j += 1024) v[j] *= r;
}

// Z = sign(T) u v^T (sign(t) = -1 for t < 0, else +1); U = T - Z; with S
// given, also the int8 signs.
__global__ __launch_bounds__(256) void k_project(const float* T, int32_t rows, int32_t cols,
                                                 const float* u, const float* v, float* Z, float* U,
                                                 int8_t* S) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)rows * cols) return;
  const int64_t i = id / cols, j = id - i * cols;
  const float t = T[id];
  const float z = (t < 0.0f ? -1.0f : 1.0f) * u[i] * v[j];
  Z[id] = z;
  if (U != nullptr) U[id] = t - z;
  if (S != nullptr) S[id] = t < 0.0f ? (int8_t)-1 : (int8_t)1;
}

// Sum of squares of (W - P) (or of W when P is null): per-workgroup partial
// sums over row blocks of 16 rows, then k_sum_parts adds them in order.
__global__ __launch_bounds__(256) void k_sumsq(const float* W, int64_t ldw, const float* P,
                                               int32_t rows, int32_t cols, float* part) {
  const int r0 = blockIdx.x * 16, r1 = min(rows, r0 + 16);
  float ss = 0.0f;
  for (int i = r0; i < r1; ++i)
    for (int j = threadIdx.x; j < cols; j += 256) {
      const float d = W[(int64_t)i * ldw + j] - (P != nullptr ? P[(int64_t)i * cols + j] : 0.0f);
      ss += d * d;
    }
  __shared__ float red[256];
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(1024) void k_sum_parts(const float* part, int32_t n, float* sc,
                                                    int slot) {
  float ss = 0.0f;
  for (int i = threadIdx.x; i < n; i += 1024) ss += part[i];
  const float t = block_sum(ss);
  if (threadIdx.x == 0) sc[slot] = t;
}

__global__ void k_rel_err(const float* sc, float* out) { *out = sqrtf(sc[kErr] / sc[kWn]); }

// fp16 scales: alpha = a, beta = m * r, gamma = b
__global__ __launch_bounds__(256) void k_scales(const float* a, int32_t N, const float* m,
                                                const float* r, int32_t k, const float* b,
                                                int32_t M, half_t* alpha, half_t* beta,
                                                half_t* gamma) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id < N) alpha[id] = (half_t)a[id];
  if (id < k) beta[id] = (half_t)(m[id] * r[id]);
  if (id < M) gamma[id] = (half_t)b[id];
}

inline unsigned blocks(int64_t n, int per = 256) { return (unsigned)cdiv(n, per); }

}  // namespace

FactorLayout factor_layout(int64_t N, int64_t M, int64_t k) {
  FactorLayout L{};
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off += align256(floats * sizeof(float));
    return o;
  };
  const int64_t big = N > M ? N : M;
  L.xa = take(N * k);
  L.za = take(N * k);
  L.ua = take(N * k);
  L.xb = take(k * M);
  L.zb = take(k * M);
  L.ub = take(k * M);
  L.base = take(big * k);
  L.rhs = take(big * k);
  L.g = take(k * k);
  L.inv = take(k * k);
  L.inv2 = take(k * k);
  L.t = take(k * k);
  L.ua_vec = take(N);
  L.va_vec = take(k);
  L.ub_vec = take(k);
  L.vb_vec = take(M);
  // power-iteration partial sums: side A (N rows, k columns) and side B (k
  // rows, M columns)
  // (also the k column sums of the regularised Gram matrix and the cdiv(N,
  // 16) partial sums of the error check)
  const int64_t pa = cdiv(N, kRowChunk) * k, pb = cdiv(k, kRowChunk) * M;
  int64_t pmax = pa > pb ? pa : pb;
  if (pmax < k) pmax = k;
  if (pmax < cdiv(N, 16)) pmax = cdiv(N, 16);
  L.part = take(pmax);
  L.prod = take(N * M);
  L.sc = take(kNScalars);
  L.total = off;
  return L;
}

hipError_t launch_factorize(const FactorArgs& a, hipStream_t s) {
  const FactorLayout L = factor_layout(a.N, a.M, a.k);
  char* ws = (char*)a.ws;
  auto F = [&](size_t off) { return (float*)(ws + off); };
  float *XA = F(L.xa), *ZA = F(L.za), *UA = F(L.ua), *XB = F(L.xb), *ZB = F(L.zb),
        *UB = F(L.ub), *base = F(L.base), *rhs = F(L.rhs), *G = F(L.g), *inv = F(L.inv),
        *inv2 = F(L.inv2), *T = F(L.t), *ua = F(L.ua_vec), *va = F(L.va_vec), *ub = F(L.ub_vec),
        *vb = F(L.vb_vec), *part = F(L.part), *prod = F(L.prod), *sc = F(L.sc);
  const int64_t N = a.N, M = a.M, k = a.k;
  const int n_ns = 2 * (int)ceil(log2((double)k + 1.0)) + 10;
  hipError_t e;
#define DBF_TRY(x) \
  if ((e = (x)) != hipSuccess) return e
#define DBF_LAUNCH(kern, grid, block, ...)                             \
  do {                                                                 \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, s, __VA_ARGS__); \
    DBF_TRY(hipGetLastError());                                        \
  } while (0)

  // SVID of T (rows x cols) in place of Z (and U = T - Z when U is given):
  // power iteration for the top singular pair of |T| from the current v.
  auto svid = [&](float* Tm, int64_t rows, int64_t cols, float* u, float* v, float* Z, float* U,
                  int8_t* S, int iters) -> hipError_t {
    const int32_t n_chunks = (int32_t)cdiv(rows, kRowChunk);
    for (int it = 0; it < iters; ++it) {
      DBF_LAUNCH(k_absmv_rows, blocks(rows, 4), 256, (const float*)Tm, (int32_t)rows,
                 (int32_t)cols, (const float*)v, u);
      DBF_LAUNCH(k_absmv_cols, (unsigned)(cdiv(cols, 64) * n_chunks), 256, (const float*)Tm,
                 (int32_t)rows, (int32_t)cols, (const float*)u, part);
      DBF_LAUNCH(k_norm_cols, 1, 1024, (const float*)part, n_chunks, (int32_t)cols, v);
    }
    DBF_LAUNCH(k_absmv_rows, blocks(rows, 4), 256, (const float*)Tm, (int32_t)rows, (int32_t)cols,
               (const float*)v, u);
    DBF_LAUNCH(k_split, 1, 1024, u, (int32_t)rows, v, (int32_t)cols);
    DBF_LAUNCH(k_project, blocks(rows * cols), 256, (const float*)Tm, (int32_t)rows,
               (int32_t)cols, (const float*)u, (const float*)v, Z, U, S);
    return hipSuccess;
  };
  // (G + rho I)^-1 into inv (G is k x k, already formed; regularised in place)
  auto ns_inverse = [&]() -> hipError_t {
    DBF_LAUNCH(k_colabs, cdiv(k, 64), 1024, (const float*)G, (int32_t)k, a.rho0, part);
    DBF_LAUNCH(k_regularise, 1, 1024, G, (int32_t)k, a.rho0, (const float*)part, sc);
    DBF_LAUNCH(k_ns_init, blocks(k * k), 256, inv, (int32_t)k, (const float*)sc);
    float* x = inv;
    float* y = inv2;
    for (int it = 0; it < n_ns; ++it) {
      DBF_TRY((sgemm<false, false>(G, k, x, k, T, k, k, k, k, s)));  // T = A X
      DBF_LAUNCH(k_two_minus, blocks(k * k), 256, T, (int32_t)k);
      DBF_TRY((sgemm<false, false>(x, k, T, k, y, k, k, k, k, s)));  // X' = X (2I - A X)
      float* t = x;
      x = y;
      y = t;
    }
    if (x != inv) DBF_LAUNCH(k_copy, blocks(k * k), 256, inv, (const float*)x, k * k);
    return hipSuccess;
  };

  // ---- start: Y = SVID(omega W) (or the given start) ----
  const int n_pow = a.power_iters;
  DBF_LAUNCH(k_fill, blocks(k), 256, va, (int64_t)k, 1.0f);
  DBF_LAUNCH(k_fill, blocks(M), 256, vb, (int64_t)M, 1.0f);
  bool have_x = false;
  if (a.X0 != nullptr) {
    DBF_LAUNCH(k_copy, blocks(N * k), 256, ZA, a.X0, N * k);
    DBF_LAUNCH(k_copy, blocks(k * M), 256, ZB, a.Y0, k * M);
    have_x = true;
  } else {
    DBF_TRY((sgemm<false, false>(a.omega, N, a.W, a.ldw, XB, M, k, M, N, s)));  // omega W
    DBF_TRY(svid(XB, k, M, ub, vb, ZB, nullptr, nullptr, 4 * n_pow));
  }
  for (int o = 0; o < a.outer; ++o) {
    // ---- side A: Y fixed (ZB), X (N x k) ----
    DBF_TRY((sgemm<false, true>(ZB, M, ZB, M, G, k, k, k, M, s)));          // G = Y Y^T
    DBF_TRY(ns_inverse());
    DBF_TRY((sgemm<false, true>(a.W, a.ldw, ZB, M, base, k, N, k, M, s)));  // base = W Y^T
    if (!have_x) {
      // first X: SVID of the regularised least-squares solution
      DBF_TRY((sgemm<false, false>(base, k, inv, k, XA, k, N, k, k, s)));
      DBF_TRY(svid(XA, N, k, ua, va, ZA, nullptr, nullptr, 4 * n_pow));
      have_x = true;
    }
    DBF_LAUNCH(k_fill, blocks(N * k), 256, UA, N * k, 0.0f);
    for (int it = 0; it < a.admm_iters; ++it) {
      DBF_LAUNCH(k_rhs, blocks(N * k), 256, (const float*)base, (const float*)ZA, (const float*)UA,
                 rhs, N * k, (const float*)sc);
      DBF_TRY((sgemm<false, false>(rhs, k, inv, k, XA, k, N, k, k, s)));  // X = rhs (G + rho I)^-1
      DBF_LAUNCH(k_add, blocks(N * k), 256, XA, (const float*)UA, N * k);  // T = X + U
      DBF_TRY(svid(XA, N, k, ua, va, ZA, UA, nullptr, n_pow));
    }
    // ---- side B: X fixed (ZA), Y (k x M) ----
    DBF_TRY((sgemm<true, false>(ZA, k, ZA, k, G, k, k, k, N, s)));          // G = X^T X
    DBF_TRY(ns_inverse());
    DBF_TRY((sgemm<true, false>(ZA, k, a.W, a.ldw, base, M, k, M, N, s)));  // base = X^T W
    DBF_LAUNCH(k_fill, blocks(k * M), 256, UB, k * M, 0.0f);
    for (int it = 0; it < a.admm_iters; ++it) {
      DBF_LAUNCH(k_rhs, blocks(k * M), 256, (const float*)base, (const float*)ZB, (const float*)UB,
                 rhs, k * M, (const float*)sc);
      DBF_TRY((sgemm<false, false>(inv, k, rhs, M, XB, M, k, M, k, s)));  // Y = (G + rho I)^-1 rhs
      DBF_LAUNCH(k_add, blocks(k * M), 256, XB, (const float*)UB, k * M);
      DBF_TRY(svid(XB, k, M, ub, vb, ZB, UB, nullptr, n_pow));
    }
  }
  // ---- factors: one more projection of each side (exact: Z is already a
  // scaled sign matrix) gives the signs and the split scales ----
  DBF_LAUNCH(k_copy, blocks(N * k), 256, XA, (const float*)ZA, N * k);
  DBF_TRY(svid(XA, N, k, ua, va, ZA, nullptr, a.S1, 4 * n_pow));
  DBF_LAUNCH(k_copy, blocks(k * M), 256, XB, (const float*)ZB, k * M);
  DBF_TRY(svid(XB, k, M, ub, vb, ZB, nullptr, a.S2, 4 * n_pow));
  DBF_LAUNCH(k_scales, blocks(N > M ? (N > k ? N : k) : (M > k ? M : k)), 256, (const float*)ua,
             (int32_t)N, (const float*)va, (const float*)ub, (int32_t)k, (const float*)vb,
             (int32_t)M, (half_t*)a.alpha, (half_t*)a.beta, (half_t*)a.gamma);
  if (a.rel_err != nullptr) {
    DBF_TRY((sgemm<false, false>(ZA, k, ZB, M, prod, M, N, M, k, s)));
    const int32_t nrb = (int32_t)cdiv(N, 16);
    DBF_LAUNCH(k_sumsq, (unsigned)nrb, 256, a.W, a.ldw, (const float*)prod, (int32_t)N,
               (int32_t)M, part);
    DBF_LAUNCH(k_sum_parts, 1, 1024, (const float*)part, nrb, sc, (int)kErr);
    DBF_LAUNCH(k_sumsq, (unsigned)nrb, 256, a.W, a.ldw, (const float*)nullptr, (int32_t)N,
               (int32_t)M, part);
    DBF_LAUNCH(k_sum_parts, 1, 1024, (const float*)part, nrb, sc, (int)kWn);
    DBF_LAUNCH(k_rel_err, 1, 1, (const float*)sc, a.rel_err);
  }
#undef DBF_LAUNCH
#undef DBF_TRY
  return hipSuccess;
}

}  // namespace dbf
