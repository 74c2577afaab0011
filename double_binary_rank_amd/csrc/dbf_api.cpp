// C ABI of the library: synchronous argument validation, then launches on
// the caller's stream.  No allocation; the only global state is the table
// of per-GPU addresses of dbf_forward_no_alloc's static scratch array.
#include "../../include/dbf.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "dbf_launch.h"

using dbf::cdiv;

// Workspace of dbf_forward_no_alloc: one static array per GPU, part of the
// loaded code object.  In host code its name is only a stand-in; the device
// address of each GPU's copy is looked up once (hipGetSymbolAddress with that
// GPU current) and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[DBF_NO_ALLOC_SCRATCH_BYTES];

namespace {

inline bool aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }

dbf_status hip_status(hipError_t e) { return e == hipSuccess ? DBF_OK : DBF_ERR_HIP; }

bool valid_dtype_out(dbf_dtype t) { return t == DBF_F16 || t == DBF_F32; }

constexpr uint32_t kPhases = DBF_RUN_PREP | DBF_RUN_STAGE1 | DBF_RUN_STAGE2;
constexpr uint32_t kKnownFlags = DBF_ACCUMULATE | DBF_PATH_GEMV | DBF_PATH_MFMA | kPhases;

// phase bits 0 (prep), 1 (stage 1), 2 (stage 2); none selected means all
int phases_of(uint32_t flags) {
  const uint32_t f = flags & kPhases;
  if (f == 0) return 7;
  return ((f & DBF_RUN_PREP) ? 1 : 0) | ((f & DBF_RUN_STAGE1) ? 2 : 0) |
         ((f & DBF_RUN_STAGE2) ? 4 : 0);
}

// Checks shared by dbf_forward and dbf_forward_multi_adapter.
dbf_status check_common(const void* x, int64_t ldx, int64_t N, int64_t R, int64_t M, int32_t ell,
                        int64_t T, void* y, int64_t ldy, dbf_dtype y_type, uint32_t flags,
                        void* ws, size_t ws_bytes) {
  if (N <= 0 || R <= 0 || M <= 0 || ell < 1 || T < 0) return DBF_ERR_INVALID_ARG;
  if (N > DBF_MAX_DIM || R > DBF_MAX_DIM || M > DBF_MAX_DIM || T > DBF_MAX_DIM)
    return DBF_ERR_INVALID_ARG;
  if (!valid_dtype_out(y_type)) return DBF_ERR_INVALID_ARG;
  if (flags & ~kKnownFlags) return DBF_ERR_INVALID_ARG;
  if ((flags & DBF_PATH_GEMV) && (flags & DBF_PATH_MFMA)) return DBF_ERR_INVALID_ARG;
  if (T == 0) return DBF_OK;
  if (x == nullptr || y == nullptr) return DBF_ERR_INVALID_ARG;
  if (ldx < M || ldy < N) return DBF_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || (ldx % 8) != 0) return DBF_ERR_ALIGNMENT;
  if ((ldy % (y_type == DBF_F16 ? 8 : 4)) != 0) return DBF_ERR_ALIGNMENT;
  const size_t need = dbf::workspace_bytes(N, R, M, ell, T);
  if (ws == nullptr || ws_bytes < need) return DBF_ERR_WORKSPACE;
  if (!aligned16(ws)) return DBF_ERR_ALIGNMENT;
  return DBF_OK;
}

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the GPU that runs `stream`.
hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

dbf::Path pick_path(uint32_t flags, int64_t per_segment, int64_t R, int64_t M, bool multi) {
  if (flags & DBF_PATH_GEMV) return dbf::Path::Gemv;
  if (flags & DBF_PATH_MFMA) return dbf::Path::Mfma;
  return dbf::choose_path(per_segment, R, M, multi);
}

}  // namespace

extern "C" {

int32_t dbf_abi_version(void) { return DBF_ABI_VERSION; }

const char* dbf_status_string(dbf_status s) {
  switch (s) {
    case DBF_OK:
      return "DBF_OK";
    case DBF_ERR_INVALID_ARG:
      return "DBF_ERR_INVALID_ARG: null pointer, non-positive size, bad stride, dtype or flag";
    case DBF_ERR_ALIGNMENT:
      return "DBF_ERR_ALIGNMENT: a pointer or stride is not aligned as required";
    case DBF_ERR_WORKSPACE:
      return "DBF_ERR_WORKSPACE: workspace missing or smaller than dbf_workspace_bytes";
    case DBF_ERR_HIP:
      return "DBF_ERR_HIP: the HIP runtime refused a launch";
    case DBF_ERR_TOO_LARGE:
      return "DBF_ERR_TOO_LARGE: the call needs a larger workspace than the library's static "
             "scratch array (DBF_NO_ALLOC_SCRATCH_BYTES); use dbf_forward with a workspace";
    default:
      return "unknown dbf_status";
  }
}

dbf_status dbf_packed_bytes(int64_t rows, int64_t cols, size_t* bytes) {
  if (rows <= 0 || cols <= 0 || bytes == nullptr) return DBF_ERR_INVALID_ARG;
  *bytes = (size_t)dbf::packed_words_total(rows, cols) * 4u;
  return DBF_OK;
}

dbf_status dbf_pack_signs(const void* src, dbf_dtype src_type, int64_t rows, int64_t cols,
                          int64_t ld_src, uint32_t* dst, void* stream) {
  if (src == nullptr || dst == nullptr || rows <= 0 || cols <= 0 || ld_src < cols)
    return DBF_ERR_INVALID_ARG;
  if (src_type != DBF_I8 && src_type != DBF_F16 && src_type != DBF_F32) return DBF_ERR_INVALID_ARG;
  if (!aligned16(dst)) return DBF_ERR_ALIGNMENT;
  return hip_status(
      dbf::launch_pack(src, (int)src_type, rows, cols, ld_src, dst, (hipStream_t)stream));
}

dbf_status dbf_unpack_signs(const uint32_t* src, int64_t rows, int64_t cols, int8_t* dst,
                            int64_t ld_dst, void* stream) {
  if (src == nullptr || dst == nullptr || rows <= 0 || cols <= 0 || ld_dst < cols)
    return DBF_ERR_INVALID_ARG;
  if (!aligned16(src)) return DBF_ERR_ALIGNMENT;
  return hip_status(dbf::launch_unpack(src, rows, cols, dst, ld_dst, (hipStream_t)stream));
}

dbf_status dbf_transpose_signs(const uint32_t* src, int64_t rows, int64_t cols, uint32_t* dst,
                               void* stream) {
  if (src == nullptr || dst == nullptr || rows <= 0 || cols <= 0 || rows > DBF_MAX_DIM ||
      cols > DBF_MAX_DIM)
    return DBF_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst)) return DBF_ERR_ALIGNMENT;
  if (src == dst) return DBF_ERR_INVALID_ARG;
  return hip_status(dbf::launch_transpose(src, rows, cols, dst, (hipStream_t)stream));
}

dbf_status dbf_workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T,
                               size_t* bytes) {
  if (N <= 0 || R <= 0 || M <= 0 || ell < 1 || T < 0 || bytes == nullptr)
    return DBF_ERR_INVALID_ARG;
  *bytes = dbf::workspace_bytes(N, R, M, ell, T);
  return DBF_OK;
}

dbf_status dbf_forward(const void* x, int64_t ldx, const uint32_t* B1, const uint32_t* B2,
                       const void* alpha, const void* beta, const void* gamma, int64_t N,
                       int64_t R, int64_t M, int32_t ell, int64_t T, void* y, int64_t ldy,
                       dbf_dtype y_type, uint32_t flags, void* ws, size_t ws_bytes,
                       void* stream) {
  if (B1 == nullptr || B2 == nullptr || alpha == nullptr || beta == nullptr || gamma == nullptr)
    return DBF_ERR_INVALID_ARG;
  dbf_status st = check_common(x, ldx, N, R, M, ell, T, y, ldy, y_type, flags, ws, ws_bytes);
  if (st != DBF_OK || T == 0) return st;
  if (!aligned16(B1) || !aligned16(B2)) return DBF_ERR_ALIGNMENT;
  if ((((uintptr_t)alpha) | ((uintptr_t)beta) | ((uintptr_t)gamma)) & 1u) return DBF_ERR_ALIGNMENT;

  dbf::ForwardArgs a{};
  a.x = (const dbf::half_t*)x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = (y_type == DBF_F32);
  a.accumulate = (flags & DBF_ACCUMULATE) != 0;
  a.N = N;
  a.R = R;
  a.M = M;
  a.T = T;
  a.ell = ell;
  a.single = dbf::Factors{B1, B2, (const dbf::half_t*)alpha, (const dbf::half_t*)beta,
                          (const dbf::half_t*)gamma};
  a.multi = false;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  a.path = pick_path(flags, T, R, M, false);
  a.phases = phases_of(flags);
  return hip_status(dbf::launch_forward(a, (hipStream_t)stream));
}

dbf_status dbf_forward_no_alloc(const void* x, int64_t ldx, const uint32_t* B1,
                                const uint32_t* B2, const void* alpha, const void* beta,
                                const void* gamma, int64_t N, int64_t R, int64_t M, int32_t ell,
                                int64_t T, void* y, int64_t ldy, dbf_dtype y_type,
                                uint32_t flags, void* stream) {
  if (N <= 0 || R <= 0 || M <= 0 || ell < 1 || T < 0 || N > DBF_MAX_DIM || R > DBF_MAX_DIM ||
      M > DBF_MAX_DIM || T > DBF_MAX_DIM)
    return DBF_ERR_INVALID_ARG;
  if (T == 0) return DBF_OK;
  if (dbf::workspace_bytes(N, R, M, ell, T) > DBF_NO_ALLOC_SCRATCH_BYTES) return DBF_ERR_TOO_LARGE;
  void* ws = nullptr;
  const hipError_t e = scratch_address((hipStream_t)stream, &ws);
  if (e != hipSuccess) return DBF_ERR_HIP;
  return dbf_forward(x, ldx, B1, B2, alpha, beta, gamma, N, R, M, ell, T, y, ldy, y_type, flags,
                     ws, DBF_NO_ALLOC_SCRATCH_BYTES, stream);
}

dbf_status dbf_forward_multi_adapter(const void* x, int64_t ldx, int64_t T, const int32_t* ids,
                                     int32_t num_adapters, const uint32_t* const* B1s,
                                     const uint32_t* const* B2s, const void* const* alphas,
                                     const void* const* betas, const void* const* gammas,
                                     int64_t N, int64_t R, int64_t M, int32_t ell, void* y,
                                     int64_t ldy, dbf_dtype y_type, uint32_t flags, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (num_adapters < 1 || B1s == nullptr || B2s == nullptr || alphas == nullptr ||
      betas == nullptr || gammas == nullptr)
    return DBF_ERR_INVALID_ARG;
  dbf_status st = check_common(x, ldx, N, R, M, ell, T, y, ldy, y_type, flags, ws, ws_bytes);
  if (st != DBF_OK || T == 0) return st;
  if (ids == nullptr) return DBF_ERR_INVALID_ARG;
  if ((((uintptr_t)B1s) | ((uintptr_t)B2s) | ((uintptr_t)alphas) | ((uintptr_t)betas) |
       ((uintptr_t)gammas)) & 7u)
    return DBF_ERR_ALIGNMENT;
  if (((uintptr_t)ids) & 3u) return DBF_ERR_ALIGNMENT;

  dbf::ForwardArgs a{};
  a.x = (const dbf::half_t*)x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = (y_type == DBF_F32);
  a.accumulate = (flags & DBF_ACCUMULATE) != 0;
  a.N = N;
  a.R = R;
  a.M = M;
  a.T = T;
  a.ell = ell;
  a.multi = true;
  a.ids = ids;
  a.num_adapters = num_adapters;
  a.B1s = B1s;
  a.B2s = B2s;
  a.alphas = (const dbf::half_t* const*)alphas;
  a.betas = (const dbf::half_t* const*)betas;
  a.gammas = (const dbf::half_t* const*)gammas;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  const int64_t per = T / (num_adapters < T ? num_adapters : T);
  a.path = pick_path(flags, per, R, M, true);
  a.phases = phases_of(flags);
  return hip_status(dbf::launch_forward(a, (hipStream_t)stream));
}

dbf_status dbf_grouped_workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T,
                                       int32_t num_layers, size_t* bytes) {
  if (N <= 0 || R <= 0 || M <= 0 || ell < 1 || T < 0 || bytes == nullptr) return DBF_ERR_INVALID_ARG;
  if (num_layers < 1 || num_layers > dbf::kMaxGroup) return DBF_ERR_INVALID_ARG;
  *bytes = (size_t)num_layers * dbf::align256(dbf::workspace_bytes(N, R, M, ell, T));
  return DBF_OK;
}

dbf_status dbf_forward_grouped(const void* x, int64_t ldx, int64_t T, int32_t num_layers,
                               const uint32_t* const* B1s, const uint32_t* const* B2s,
                               const void* const* alphas, const void* const* betas,
                               const void* const* gammas, int64_t N, int64_t R, int64_t M,
                               int32_t ell, void* y, int64_t ldy, int64_t y_layer_stride,
                               dbf_dtype y_type, uint32_t flags, void* ws, size_t ws_bytes,
                               void* stream) {
  if (num_layers < 1 || num_layers > dbf::kMaxGroup || B1s == nullptr || B2s == nullptr ||
      alphas == nullptr || betas == nullptr || gammas == nullptr)
    return DBF_ERR_INVALID_ARG;
  const size_t layer_ws = dbf::align256(dbf::workspace_bytes(N > 0 ? N : 1, R > 0 ? R : 1,
                                                             M > 0 ? M : 1, ell > 0 ? ell : 1,
                                                             T > 0 ? T : 0));
  // per-layer checks as for dbf_forward, on layer 0's slice of the workspace
  dbf_status st = check_common(x, ldx, N, R, M, ell, T, y, ldy, y_type, flags, ws,
                               ws_bytes / (size_t)num_layers);
  if (st != DBF_OK || T == 0) return st;
  if (ws_bytes < layer_ws * (size_t)num_layers) return DBF_ERR_WORKSPACE;
  const int64_t esz = y_type == DBF_F32 ? 4 : 2;
  if (num_layers > 1 && y_layer_stride < ldy * (T - 1) + N) return DBF_ERR_INVALID_ARG;
  if ((y_layer_stride * esz) % 16 != 0) return DBF_ERR_ALIGNMENT;
  dbf::ForwardArgs a{};
  for (int j = 0; j < num_layers; ++j) {
    if (B1s[j] == nullptr || B2s[j] == nullptr || alphas[j] == nullptr || betas[j] == nullptr ||
        gammas[j] == nullptr)
      return DBF_ERR_INVALID_ARG;
    if (!aligned16(B1s[j]) || !aligned16(B2s[j])) return DBF_ERR_ALIGNMENT;
    if ((((uintptr_t)alphas[j]) | ((uintptr_t)betas[j]) | ((uintptr_t)gammas[j])) & 1u)
      return DBF_ERR_ALIGNMENT;
    a.grp[j] = dbf::Factors{B1s[j], B2s[j], (const dbf::half_t*)alphas[j],
                            (const dbf::half_t*)betas[j], (const dbf::half_t*)gammas[j]};
  }
  a.x = (const dbf::half_t*)x;
  a.ldx = ldx;
  a.y = y;
  a.ldy = ldy;
  a.y_f32 = (y_type == DBF_F32);
  a.accumulate = (flags & DBF_ACCUMULATE) != 0;
  a.N = N;
  a.R = R;
  a.M = M;
  a.T = T;
  a.ell = ell;
  a.multi = false;
  a.ws = ws;
  a.ws_bytes = layer_ws;
  a.path = pick_path(flags, T, R, M, false);
  a.phases = phases_of(flags);
  a.group = num_layers;
  a.y_layer_bytes = y_layer_stride * esz;
  a.layer_ws = layer_ws;
  return hip_status(dbf::launch_forward_grouped(a, (hipStream_t)stream));
}

dbf_status dbf_backward_workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T,
                                        size_t* bytes) {
  if (N <= 0 || R <= 0 || M <= 0 || ell < 1 || T <= 0 || bytes == nullptr)
    return DBF_ERR_INVALID_ARG;
  if (N > DBF_MAX_DIM || R > DBF_MAX_DIM || M > DBF_MAX_DIM || T > DBF_MAX_DIM)
    return DBF_ERR_INVALID_ARG;
  *bytes = dbf::bwd_layout(N, R, M, ell, T).total;
  return DBF_OK;
}

dbf_status dbf_backward(const void* x, int64_t ldx, const void* g, int64_t ldg, const uint32_t* B1,
                        const uint32_t* B2, const uint32_t* B1t, const uint32_t* B2t,
                        const void* alpha, const void* beta, const void* gamma, int64_t N,
                        int64_t R, int64_t M, int32_t ell, int64_t T, void* dx, int64_t lddx,
                        dbf_dtype dx_type, float* dalpha, float* dbeta, float* dgamma, float* dS1,
                        float* dS2, const float* H1, const float* H2, float tau, float* dH1,
                        float* dH2, void* ws, size_t ws_bytes, void* stream) {
  if (N <= 0 || R <= 0 || M <= 0 || ell < 1 || T <= 0) return DBF_ERR_INVALID_ARG;
  if (N > DBF_MAX_DIM || R > DBF_MAX_DIM || M > DBF_MAX_DIM || T > DBF_MAX_DIM)
    return DBF_ERR_INVALID_ARG;
  // the feature-major tiles index the tokens of all terms with 32 bits
  if ((int64_t)ell * cdiv(T, 128) * 128 > INT32_MAX) return DBF_ERR_INVALID_ARG;
  if (x == nullptr || g == nullptr || B1 == nullptr || B2 == nullptr || B1t == nullptr ||
      B2t == nullptr || alpha == nullptr || beta == nullptr || gamma == nullptr || dx == nullptr ||
      dalpha == nullptr || dbeta == nullptr || dgamma == nullptr)
    return DBF_ERR_INVALID_ARG;
  if ((H1 == nullptr) != (dH1 == nullptr) || (H2 == nullptr) != (dH2 == nullptr))
    return DBF_ERR_INVALID_ARG;
  if ((H1 != nullptr || H2 != nullptr) && !(tau > 0.0f && tau < 3.0e38f)) return DBF_ERR_INVALID_ARG;
  if (dx_type != DBF_F16 && dx_type != DBF_F32) return DBF_ERR_INVALID_ARG;
  if (ldx < M || ldg < N || lddx < M) return DBF_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(g) || (ldx % 8) != 0 || (ldg % 8) != 0)
    return DBF_ERR_ALIGNMENT;
  if (!aligned16(B1) || !aligned16(B2) || !aligned16(B1t) || !aligned16(B2t))
    return DBF_ERR_ALIGNMENT;
  if ((((uintptr_t)alpha) | ((uintptr_t)beta) | ((uintptr_t)gamma)) & 1u) return DBF_ERR_ALIGNMENT;
  if ((((uintptr_t)dx) & (dx_type == DBF_F32 ? 3u : 1u)) != 0) return DBF_ERR_ALIGNMENT;
  if ((((uintptr_t)dalpha) | ((uintptr_t)dbeta) | ((uintptr_t)dgamma) | ((uintptr_t)dS1) |
       ((uintptr_t)dS2) | ((uintptr_t)H1) | ((uintptr_t)H2) | ((uintptr_t)dH1) | ((uintptr_t)dH2)) &
      3u)
    return DBF_ERR_ALIGNMENT;
  if (ws == nullptr || ws_bytes < dbf::bwd_layout(N, R, M, ell, T).total) return DBF_ERR_WORKSPACE;
  if (!aligned16(ws)) return DBF_ERR_ALIGNMENT;

  dbf::BackwardArgs a{};
  a.x = (const dbf::half_t*)x;
  a.ldx = ldx;
  a.g = (const dbf::half_t*)g;
  a.ldg = ldg;
  a.B1 = B1;
  a.B2 = B2;
  a.B1t = B1t;
  a.B2t = B2t;
  a.alpha = (const dbf::half_t*)alpha;
  a.beta = (const dbf::half_t*)beta;
  a.gamma = (const dbf::half_t*)gamma;
  a.N = N;
  a.R = R;
  a.M = M;
  a.T = T;
  a.ell = ell;
  a.dx = dx;
  a.lddx = lddx;
  a.dx_f32 = (dx_type == DBF_F32);
  a.dalpha = dalpha;
  a.dbeta = dbeta;
  a.dgamma = dgamma;
  a.dS1 = dS1;
  a.dS2 = dS2;
  a.H1 = H1;
  a.H2 = H2;
  a.tau = tau;
  a.dH1 = dH1;
  a.dH2 = dH2;
  a.ws = ws;
  return hip_status(dbf::launch_backward(a, (hipStream_t)stream));
}

dbf_status dbf_factorize_workspace_bytes(int64_t N, int64_t M, int64_t k, size_t* bytes) {
  if (N <= 0 || M <= 0 || k <= 0 || bytes == nullptr) return DBF_ERR_INVALID_ARG;
  if (N > DBF_MAX_DIM || M > DBF_MAX_DIM || k > DBF_MAX_DIM) return DBF_ERR_INVALID_ARG;
  *bytes = dbf::factor_layout(N, M, k).total;
  return DBF_OK;
}

dbf_status dbf_factorize(const float* W, int64_t N, int64_t M, int64_t ldw, int64_t k,
                         const float* omega, const float* X0, const float* Y0, int32_t outer,
                         int32_t admm_iters, int32_t power_iters, float rho0, int8_t* S1,
                         int8_t* S2, void* alpha, void* beta, void* gamma, float* rel_err,
                         void* ws, size_t ws_bytes, void* stream) {
  if (N <= 0 || M <= 0 || k <= 0) return DBF_ERR_INVALID_ARG;
  if (N > DBF_MAX_DIM || M > DBF_MAX_DIM || k > DBF_MAX_DIM) return DBF_ERR_INVALID_ARG;
  // the dense products index their tiles and rows with 32 bits
  if (cdiv(N, 64) * cdiv(M, 64) > INT32_MAX || cdiv(N > M ? N : M, 64) * cdiv(k, 64) > INT32_MAX)
    return DBF_ERR_INVALID_ARG;
  if (W == nullptr || S1 == nullptr || S2 == nullptr || alpha == nullptr || beta == nullptr ||
      gamma == nullptr)
    return DBF_ERR_INVALID_ARG;
  if (omega == nullptr && (X0 == nullptr || Y0 == nullptr)) return DBF_ERR_INVALID_ARG;
  if ((X0 == nullptr) != (Y0 == nullptr)) return DBF_ERR_INVALID_ARG;
  if (ldw < M || outer < 0 || admm_iters < 1 || power_iters < 1) return DBF_ERR_INVALID_ARG;
  if (!(rho0 > 0.0f && rho0 < 3.0e38f)) return DBF_ERR_INVALID_ARG;
  if ((((uintptr_t)W) | ((uintptr_t)omega) | ((uintptr_t)X0) | ((uintptr_t)Y0) |
       ((uintptr_t)rel_err)) & 3u)
    return DBF_ERR_ALIGNMENT;
  if ((((uintptr_t)alpha) | ((uintptr_t)beta) | ((uintptr_t)gamma)) & 1u) return DBF_ERR_ALIGNMENT;
  if (ws == nullptr || ws_bytes < dbf::factor_layout(N, M, k).total) return DBF_ERR_WORKSPACE;
  if (!aligned16(ws)) return DBF_ERR_ALIGNMENT;
  dbf::FactorArgs a{};
  a.W = W;
  a.ldw = ldw;
  a.N = N;
  a.M = M;
  a.k = k;
  a.omega = omega;
  a.X0 = X0;
  a.Y0 = Y0;
  a.outer = outer;
  a.admm_iters = admm_iters;
  a.power_iters = power_iters;
  a.rho0 = rho0;
  a.S1 = S1;
  a.S2 = S2;
  a.alpha = alpha;
  a.beta = beta;
  a.gamma = gamma;
  a.rel_err = rel_err;
  a.ws = ws;
  return hip_status(dbf::launch_factorize(a, (hipStream_t)stream));
}

}  // extern "C"
