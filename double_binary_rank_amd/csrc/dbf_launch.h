// Launchers shared by the C-ABI layer and the kernels (internal).
#pragma once

#include "dbf_common.h"

namespace dbf {

// Which kernel family evaluates the two sign-accumulation stages.
enum class Path : int { Gemv = 0, Mfma = 1 };

// Largest number of same-input layers in one grouped call.
constexpr int kMaxGroup = 8;

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
  int phases;  // bit 0: prep (operands of stage 1), bit 1: stage 1 (z), bit 2: stage 2 (y)
  // grouped same-input layers (group > 1): layer j has factors grp[j], writes
  // y + j * y_layer_bytes and uses ws + j * layer_ws
  int32_t group;
  Factors grp[kMaxGroup];
  int64_t y_layer_bytes;
  size_t layer_ws;
};

// Largest batch the small-T (fp4 matrix-core) path accepts; its operand
// buffers in the workspace are sized for this many tokens.
constexpr int64_t kGemvMaxT = 4096;
// fp8 parts each activation is split into on the small-T path.
constexpr int kParts = 3;
// Largest number of parts a decode call's stage-1 reduction is split into
// (each part writes its own partial z; stage 2 adds them in order).
constexpr int kMaxZParts = 8;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline int64_t ldz_of(int64_t R) { return cdiv(R, 8) * 8; }
inline int64_t max_colblocks(int64_t T) { return T + cdiv(T, 16) + 1; }
// Large-T path operands v_i = gamma_i * x and z_i (fp16) in MFMA operand
// order: per term, tiles of 16 tokens x 128 reduction entries, each 4 KB =
// 4 steps x 64 lanes x 8: entry (t, r) with k = r % 128 sits at half
//   ((t/16 * nkb + r/128) * 4 + k/32) * 512 + (16 * (k/8 % 4) + t%16) * 8 + k%8
// so the 16 tokens x 32 entries a wave reads for one MFMA step are 1 KB
// contiguous.  (K = reduction length, nkb = ceil(K/128).)
inline int64_t zt_term_halfs(int64_t K, int64_t T) { return cdiv(T, 16) * cdiv(K, 128) * 2048; }

// Byte offsets of the workspace regions.
struct WsLayout {
  size_t cbl, z, v, p1o, p1s, p2o, p2s, total;
};

inline WsLayout ws_layout(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T) {
  (void)N;
  WsLayout w{};
  const int64_t tg = T < kGemvMaxT ? T : kGemvMaxT;
  // small-T operands: [ell][tg][nkb][kParts][4] x 32 bytes, plus one scale byte each
  const size_t n1 = (size_t)ell * tg * cdiv(M, kColBlock) * kParts * 4;
  const size_t n2 = (size_t)ell * tg * cdiv(R, kColBlock) * kParts * 4;
  size_t off = sizeof(WsHeader);
  w.cbl = off;
  off += align256((size_t)max_colblocks(T) * sizeof(ColBlock));
  w.z = off;
  // fp32 [ell][T][ldz] on the small-T path (for ell * T <= 2, up to
  // kMaxZParts partial sums of it, one per part of a split stage-1
  // reduction), MFMA-tiled fp16 on the large-T path
  const size_t z32 = (size_t)ell * T * ldz_of(R) * sizeof(float) *
                     ((int64_t)ell * T <= 2 ? kMaxZParts : 1);
  const size_t z16 = (size_t)ell * zt_term_halfs(R, T) * sizeof(half_t);
  off += align256(z32 > z16 ? z32 : z16);
  // large-T path: v_i = gamma_i * x, fp16 tiles like z (16 tokens x 128 cols)
  w.v = off;
  off += align256((size_t)ell * zt_term_halfs(M, T) * sizeof(half_t));
  w.p1o = off;
  off += align256(n1 * 32);
  w.p1s = off;
  off += align256(n1);
  w.p2o = off;
  off += align256(n2 * 32);
  w.p2s = off;
  off += align256(n2);
  w.total = off;
  return w;
}

size_t workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T);
hipError_t launch_pack(const void* src, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       uint32_t* dst, hipStream_t s);
hipError_t launch_unpack(const uint32_t* src, int64_t rows, int64_t cols, int8_t* dst, int64_t ld,
                         hipStream_t s);
hipError_t launch_transpose(const uint32_t* src, int64_t rows, int64_t cols, uint32_t* dst,
                            hipStream_t s);
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s);
hipError_t launch_forward_grouped(const ForwardArgs& a, hipStream_t s);
Path choose_path(int64_t tokens_per_segment_estimate, int64_t R, int64_t M, bool multi);
// tokens per column block on the small-T path (3 fp8 parts x ell terms
// x tokens must fit the 16 columns of one MFMA); 0 if ell is too large.
inline int gemv_tokens_per_block(int32_t ell) { return ell <= 5 ? 16 / (kParts * ell) : 0; }
hipError_t launch_gemv(const ForwardArgs& a, hipStream_t s);
// large-T path: fp16 matrix-core contractions; with several adapters the
// column blocks hold at most kGemmChunk tokens of one adapter
constexpr int kGemmChunk = 32;
hipError_t launch_gemm(const ForwardArgs& a, hipStream_t s);
// large-T path of one adapter (not grouped): token tiles shared through LDS;
// z as fp16 rows [ell][T][ldz_of(R)] in the workspace's z region
hipError_t launch_tile_forward(const ForwardArgs& a, hipStream_t s);
bool tile_path_fits(const ForwardArgs& a);
// Token-major fp16 operand tiles (the large-T layout above) of
// scale_i[k] * src[t][k] for each of ell terms (src fp16 [T][ld], shared),
// for two sources in one launch.
struct TilesF16 {
  const half_t* src;
  int64_t ld, K;
  const half_t* scale;  // [ell][K]
  half_t* out;
};
hipError_t launch_tiles_f16_pair(const TilesF16& a, const TilesF16& b, int64_t T, int32_t ell,
                                 hipStream_t s);
// Raw per-term sign products out[i][t][r] = sum_k S[r][k] * tiles_i[t][k]
// (fp32, [ell][T][ldo]); S is a packed rows x K sign matrix.
hipError_t launch_sign_product(const uint32_t* S, int64_t rows, int64_t K, int32_t ell, int64_t T,
                               const half_t* tiles, float* out, int64_t ldo, hipStream_t s);
// Two such products of one shape in one launch (S0 with tiles0 into out0, S1
// with tiles1 into out1).
hipError_t launch_sign_product_pair(const uint32_t* S0, const uint32_t* S1, int64_t rows,
                                    int64_t K, int32_t ell, int64_t T, const half_t* tiles0,
                                    const half_t* tiles1, float* out0, float* out1, int64_t ldo,
                                    hipStream_t s);

// ------------------------------------------------------------ backward ----
struct BackwardArgs {
  const half_t* x;  // [T][ldx]
  int64_t ldx;
  const half_t* g;  // upstream gradient dL/dy, [T][ldg]
  int64_t ldg;
  const uint32_t* B1;   // N x R, packed along R
  const uint32_t* B2;   // R x M, packed along M
  const uint32_t* B1t;  // R x N, packed along N (transpose of B1)
  const uint32_t* B2t;  // M x R, packed along R (transpose of B2)
  const half_t* alpha;
  const half_t* beta;
  const half_t* gamma;
  int64_t N, R, M, T;
  int32_t ell;
  void* dx;
  int64_t lddx;
  bool dx_f32;
  float* dalpha;  // [ell][N]
  float* dbeta;   // [ell][R]
  float* dgamma;  // [ell][M]
  float* dS1;     // [N][R] or null
  float* dS2;     // [R][M] or null
  const float* H1;  // latents [N][R], [R][M], or null
  const float* H2;
  float tau;
  float* dH1;
  float* dH2;
  void* ws;
};

// Byte offsets of the backward workspace regions.
struct BwdLayout {
  size_t vt, gt, u, p, zt, pt, w, q, gf, zf, pf, vf, part, total;
};

// Tokens per chunk of the column dot products (partial sums per chunk, then
// summed over the chunks in order).
constexpr int kColdotChunk = 32;

// Reduction length of the feature-major tiles: the ell terms' tokens, each
// term padded to a multiple of 128.
inline int64_t bwd_kf(int32_t ell, int64_t T) { return (int64_t)ell * cdiv(T, 128) * 128; }
// Row stride of the fp32 intermediates U, P ([T][R]), W ([T][N]), Q ([T][M]):
// a multiple of 4 floats, for the 16-byte stores of the sign-product kernel.
inline int64_t bwd_ld(int64_t cols) { return cdiv(cols, 4) * 4; }

inline int64_t bwd_colmax(int64_t N, int64_t R, int64_t M) {
  return N > R ? (N > M ? N : M) : (R > M ? R : M);
}

inline BwdLayout bwd_layout(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const int64_t kf = bwd_kf(ell, T);
  L.vt = take((size_t)ell * zt_term_halfs(M, T) * sizeof(half_t));
  L.gt = take((size_t)ell * zt_term_halfs(N, T) * sizeof(half_t));
  L.u = take((size_t)ell * T * bwd_ld(R) * sizeof(float));
  L.p = take((size_t)ell * T * bwd_ld(R) * sizeof(float));
  L.zt = take((size_t)ell * zt_term_halfs(R, T) * sizeof(half_t));
  L.pt = take((size_t)ell * zt_term_halfs(R, T) * sizeof(half_t));
  L.w = take((size_t)ell * T * bwd_ld(N) * sizeof(float));
  L.q = take((size_t)ell * T * bwd_ld(M) * sizeof(float));
  L.gf = take((size_t)cdiv(N, 16) * kf * 16 * sizeof(half_t));
  L.zf = take((size_t)cdiv(R, 16) * kf * 16 * sizeof(half_t));
  L.pf = take((size_t)cdiv(R, 16) * kf * 16 * sizeof(half_t));
  L.vf = take((size_t)cdiv(M, 16) * kf * 16 * sizeof(half_t));
  // per-chunk partial sums of the three column dot products (dalpha,
  // dbeta, dgamma), one third each
  L.part = take((size_t)3 * cdiv(T, kColdotChunk) * ell * bwd_colmax(N, R, M) * sizeof(float));
  L.total = off;
  return L;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);

// ------------------------------------------------------- factorisation ----
struct FactorArgs {
  const float* W;  // [N][ldw]
  int64_t ldw;
  int64_t N, M, k;
  const float* omega;  // [k][N] sketch for the start, or null with X0/Y0
  const float* X0;     // [N][k] and [k][M] scaled sign start, or null
  const float* Y0;
  int32_t outer, admm_iters, power_iters;
  float rho0;
  int8_t* S1;  // [N][k]
  int8_t* S2;  // [k][M]
  void* alpha;  // fp16 [N], [k], [M]
  void* beta;
  void* gamma;
  float* rel_err;  // device scalar or null
  void* ws;
};

struct FactorLayout {
  size_t xa, za, ua, xb, zb, ub, base, rhs, g, inv, inv2, t, ua_vec, va_vec, ub_vec, vb_vec, part,
      prod, sc, total;
};

FactorLayout factor_layout(int64_t N, int64_t M, int64_t k);
hipError_t launch_factorize(const FactorArgs& a, hipStream_t s);

// large-T path of several adapters with R <= 64 and at most two terms: one
// launch per stage over 16-token tiles, z fp16 [ell][T][ldz_of(R)] in the
// workspace's z region, no prep phase
bool ma_short_fits(const ForwardArgs& a);
hipError_t launch_ma_short(const ForwardArgs& a, hipStream_t s);

}  // namespace dbf
