/*
 * dbf.h -- C ABI of the MI355X (gfx950) double-binary-factorised product.
 *
 * The operation (LoRDBA summary, section 2 "Arquitectura Central", update
 * equation; DBF summary, section 2 "Calculo en la inferencia", operation
 * order):
 *
 *     y[t] = sum_{i<ell} diag(alpha_i) . B1 . diag(beta_i) . B2 . diag(gamma_i) . x[t]
 *
 * evaluated as  scale by gamma_i -> accumulate signs of B2 -> scale by beta_i
 * -> accumulate signs of B1 -> scale by alpha_i -> sum over i.
 *
 *   x      [T][M]  fp16, row stride ldx elements (token rows)
 *   B1     N x R   signs in {-1,+1}, packed (dbf_pack_signs, cols = R)
 *   B2     R x M   signs in {-1,+1}, packed (dbf_pack_signs, cols = M)
 *   alpha  [ell][N], beta [ell][R], gamma [ell][M]   fp16, contiguous
 *   y      [T][N]  fp16 or fp32, row stride ldy elements
 *
 * The signs are shared by the ell terms; only the scales carry the term
 * index (the LoRDBA update indexes only alpha, beta, gamma).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates or frees memory and keeps no per-call state (the one
 *    exception, dbf_forward_no_alloc, uses a static device array that is
 *    part of the loaded library).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  Buffers must stay valid until the stream reaches the work.
 *    Calls are re-entrant; concurrent calls must not share a workspace.
 *  - Arguments are validated synchronously on the host before any launch;
 *    a failed check returns an error and enqueues nothing.
 *  - Sizes are element counts unless stated otherwise.
 */
#ifndef DBF_H_
#define DBF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dbf_status;
#define DBF_OK 0
#define DBF_ERR_INVALID_ARG (-1) /* null pointer, bad size/stride/dtype/flag */
#define DBF_ERR_ALIGNMENT (-2)   /* pointer or stride misaligned            */
#define DBF_ERR_WORKSPACE (-3)   /* workspace missing or too small          */
#define DBF_ERR_HIP (-4)         /* the HIP runtime refused a launch        */
#define DBF_ERR_TOO_LARGE (-5)   /* dbf_forward_no_alloc: the call needs more
                                    than DBF_NO_ALLOC_SCRATCH_BYTES        */

typedef int32_t dbf_dtype;
#define DBF_I8 1
#define DBF_F16 2
#define DBF_F32 3

/* flags for dbf_forward / dbf_forward_multi_adapter */
#define DBF_ACCUMULATE 1u /* y += product (unmerged adapter branch added onto
                             a base output, LoRDBA summary section 1); the
                             default overwrites y                            */
/* Without a path flag the library chooses by tokens per call, the rank R
   and the reduction M: the small-T kernels up to 2 tokens (up to 16 when
   R < 256, and up to 11 when M > 8192), the large-T kernels above.  The
   multi-adapter call takes the small-T kernels up to 16 tokens per adapter
   in use (T over min(T, num_adapters)). */
#define DBF_PATH_GEMV 2u  /* force the small-T (decode) kernels  (tuning/tests) */
#define DBF_PATH_MFMA 4u  /* force the large-T (prefill) kernels (tuning/tests) */
/* Run only some phases of one product (profiling, or overlapping other work
   between them); with none of these bits set, all three run.  A phase reads
   what the earlier phases of a call with the same arguments, workspace and
   path flag left in ws, on the same stream.
     DBF_RUN_PREP    the activation operands gamma_i * x (and, with several
                     adapters, the token runs) into ws
     DBF_RUN_STAGE1  z_i = beta_i * (B2 (gamma_i * x)) into ws
     DBF_RUN_STAGE2  y from z (the only phase that writes y)
   On the large-T path each phase is at most one kernel launch; with one
   adapter, a short reduction over M (a multiple of 8) and gamma 16-byte
   aligned, stage 1 reads x itself and DBF_RUN_PREP launches nothing.  With
   several adapters of rank R <= 64 and at most two terms (M a multiple of
   8, x and y rows 16-byte aligned), stage 1 reads x itself as well and
   DBF_RUN_PREP writes only the token runs. */
#define DBF_RUN_PREP 8u
#define DBF_RUN_STAGE1 16u
#define DBF_RUN_STAGE2 32u

#define DBF_ABI_VERSION 1

/* Largest N, R, M or T accepted by dbf_forward / dbf_forward_multi_adapter
   (the kernels index rows, columns and tokens with 32-bit integers). */
#define DBF_MAX_DIM (((int64_t)1) << 30)

/* ABI version of the loaded library (DBF_ABI_VERSION it was built with). */
int32_t dbf_abi_version(void);

/* Static, human-readable text for a status code. */
const char* dbf_status_string(dbf_status s);

/*
 * Bytes of the packed form of a rows x cols sign matrix, packed along cols
 * (the reduction dimension of its product).  One bit per sign (LoRDBA
 * summary, section 2 "Eficiencia de Almacenamiento"); rows are padded to a
 * multiple of 64 and cols to a multiple of 128, so the size is
 * ceil(rows/64) * ceil(cols/128) * 1024.  The layout itself is internal.
 * Errors: INVALID_ARG if rows <= 0, cols <= 0 or bytes == NULL.
 */
dbf_status dbf_packed_bytes(int64_t rows, int64_t cols, size_t* bytes);

/*
 * Binarise and pack: sign(h) per entry of the rows x cols source (row stride
 * ld_src elements) into `dst` (dbf_packed_bytes bytes, 16-byte aligned).
 * sign(h) = -1 for h < 0, +1 otherwise (+-0 and NaN give +1); this is the
 * forward binarisation B = sign(H) of the LoRDBA training pipeline
 * (summary section 2 "Pipeline de Entrenamiento", step 2).  An int8 source
 * is read the same way, so +-1 int8 matrices pack exactly.
 *   src_type: DBF_I8, DBF_F16 or DBF_F32.
 * Padding entries are written as +1.
 * Errors: INVALID_ARG (null pointer, rows/cols <= 0, ld_src < cols, bad
 * dtype), ALIGNMENT (dst not 16-byte aligned), HIP.
 */
dbf_status dbf_pack_signs(const void* src, dbf_dtype src_type, int64_t rows, int64_t cols,
                          int64_t ld_src, uint32_t* dst, void* stream);

/*
 * Inverse of dbf_pack_signs for inspection and tests: writes int8 +-1 into
 * dst [rows][ld_dst].  Errors as for dbf_pack_signs (ld_dst < cols is
 * INVALID_ARG; src must be 16-byte aligned).
 */
dbf_status dbf_unpack_signs(const uint32_t* src, int64_t rows, int64_t cols, int8_t* dst,
                            int64_t ld_dst, void* stream);

/*
 * Transpose packed signs: from the packed rows x cols matrix S in `src`
 * (dbf_pack_signs layout) write the packed cols x rows matrix S^T into `dst`
 * (dbf_packed_bytes(cols, rows) bytes).  Device buffers, 16-byte aligned,
 * not overlapping; asynchronous on `stream`.
 *
 * The transpose of the update, dW^T = sum_i diag(gamma_i) S2^T diag(beta_i)
 * S1^T diag(alpha_i), is again a double-binary product (LoRDBA summary,
 * section 2 "Arquitectura Central", with the roles of the two sign matrices
 * and of alpha and gamma exchanged).  Applied to an output gradient g it is
 * the input gradient of the training pipeline's backward pass (same summary,
 * "Pipeline de Entrenamiento", step 3): dbf_forward with B1 = S2^T (M x R),
 * B2 = S1^T (R x N), alpha = gamma, beta = beta, gamma = alpha and the roles
 * of N and M exchanged computes g dW, i.e. dW^T g per row of g.
 * Errors: INVALID_ARG (null pointer, rows/cols <= 0 or > DBF_MAX_DIM,
 * src == dst), ALIGNMENT, HIP.
 */
dbf_status dbf_transpose_signs(const uint32_t* src, int64_t rows, int64_t cols, uint32_t* dst,
                               void* stream);

/*
 * Workspace bytes needed by dbf_forward and dbf_forward_multi_adapter for
 * these sizes (the same bound serves both).  T may be 0 (returns 0 bytes
 * needed beyond a small header).
 * Errors: INVALID_ARG if N, R, M <= 0, ell < 1, T < 0 or bytes == NULL.
 */
dbf_status dbf_workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T,
                               size_t* bytes);

/*
 * y = sum_i diag(alpha_i) B1 diag(beta_i) B2 diag(gamma_i) x   for T tokens
 * (with DBF_ACCUMULATE: y += ...).  Inputs as described at the top.
 * Precision: fp32 accumulation.  On the small-T path gamma_i*x (exact in
 * fp32) and the R-vector beta_i*u stay fp32 up to the matrix-core operand
 * encoding (three e4m3 parts per value, one power-of-two scale per 128
 * values); on the large-T path beta_i*u is rounded to fp16, and gamma_i*x
 * too unless stage 1 reads x in place (then gamma is folded into the signs
 * and the products are exact).  The fp16 output is rounded to nearest-even
 * and overflows to +-inf.
 * Alignment: x, y, B1, B2 and ws 16-byte aligned; ldx a multiple of 8;
 * ldy a multiple of 8 (fp16 y) or 4 (fp32 y).
 * T == 0 is a successful no-op (x, y and ws may then be NULL).
 * Errors: INVALID_ARG (also for N, R, M or T above DBF_MAX_DIM), ALIGNMENT,
 * WORKSPACE (ws_bytes below dbf_workspace_bytes), HIP.
 */
dbf_status dbf_forward(const void* x, int64_t ldx, const uint32_t* B1, const uint32_t* B2,
                       const void* alpha, const void* beta, const void* gamma, int64_t N,
                       int64_t R, int64_t M, int32_t ell, int64_t T, void* y, int64_t ldy,
                       dbf_dtype y_type, uint32_t flags, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * dbf_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same product, arguments and results as dbf_forward, without ws/ws_bytes.
 * The workspace is a static device array of DBF_NO_ALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held from the library's first use on
 * that GPU until the process ends; its device address is looked up once per
 * GPU (on the first call there) and no call allocates or frees anything.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or different threads without ordering)
 * race on it and give undefined results; calls ordered on one stream are
 * safe.  The array keeps the last call's contents; no part of it has to
 * start at zero.
 * Errors as for dbf_forward, plus TOO_LARGE when dbf_workspace_bytes for
 * these sizes exceeds DBF_NO_ALLOC_SCRATCH_BYTES (nothing is launched), and
 * HIP if the array's address cannot be obtained.
 */
#define DBF_NO_ALLOC_SCRATCH_BYTES (((size_t)32) << 20)
dbf_status dbf_forward_no_alloc(const void* x, int64_t ldx, const uint32_t* B1,
                                const uint32_t* B2, const void* alpha, const void* beta,
                                const void* gamma, int64_t N, int64_t R, int64_t M, int32_t ell,
                                int64_t T, void* y, int64_t ldy, dbf_dtype y_type,
                                uint32_t flags, void* stream);

/*
 * Batched adapter serving (LoRDBA summary, section 1: many unmerged adapters
 * served together, as in S-LoRA / Punica).  Token t uses adapter ids[t]:
 *   y[t] = DBF_{ids[t]}(x[t])      (with DBF_ACCUMULATE: y[t] += ...)
 * Tokens whose id is outside [0, num_adapters) contribute nothing: their row
 * of y is written as 0, or left unchanged under DBF_ACCUMULATE.
 *   ids      device int32 [T]; any order is correct, runs of equal ids are
 *            processed together (sorted ids are fastest)
 *   B1s, B2s, alphas, betas, gammas   DEVICE arrays of num_adapters device
 *            pointers, each as in dbf_forward; every adapter has the same
 *            N, R, M and ell.
 * Errors as for dbf_forward, plus INVALID_ARG for num_adapters < 1 or a
 * null table.  Adapter pointers inside the tables are not checked (they live
 * on the device).
 */
dbf_status dbf_forward_multi_adapter(const void* x, int64_t ldx, int64_t T, const int32_t* ids,
                                     int32_t num_adapters, const uint32_t* const* B1s,
                                     const uint32_t* const* B2s, const void* const* alphas,
                                     const void* const* betas, const void* const* gammas,
                                     int64_t N, int64_t R, int64_t M, int32_t ell, void* y,
                                     int64_t ldy, dbf_dtype y_type, uint32_t flags, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * Workspace bytes needed by dbf_forward_grouped: num_layers (1..8) slices,
 * each the dbf_workspace_bytes of one layer rounded up to 256 bytes.
 * Errors: INVALID_ARG as for dbf_workspace_bytes, or num_layers outside
 * 1..8.
 */
dbf_status dbf_grouped_workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T,
                                       int32_t num_layers, size_t* bytes);

/*
 * Several layers on the same input (the q/k/v or up/gate projections of a
 * decoder layer: LoRDBA summary, section 1, adapters evaluated unmerged next
 * to the base layers; decode throughput is the DBF summary's second speed
 * figure, section 4): for j < num_layers,
 *   y_j = sum_i diag(alpha_ji) B1_j diag(beta_ji) B2_j diag(gamma_ji) x
 * written to y + j * y_layer_stride elements (with DBF_ACCUMULATE added onto
 * it: the fused add into the base layers' outputs).  Every layer has the
 * same N, R, M and ell.  B1s .. gammas are HOST arrays of num_layers device
 * pointers (1 <= num_layers <= 8), each checked as in dbf_forward.  When
 * both stages of the chosen path can run every layer in one launch (the
 * decode stages that build their own operand parts; the large-T stages with
 * x read in place and a reduction of more than 2 blocks in stage 2) they
 * do, otherwise the layers run one after another; either way each layer's
 * result is bit for bit that of dbf_forward on it.
 *   y_layer_stride  elements between layers' outputs: at least
 *                   ldy * (T - 1) + N when num_layers > 1, and a multiple
 *                   of 16 bytes
 *   ws              dbf_grouped_workspace_bytes bytes
 * Errors as for dbf_forward, plus INVALID_ARG for num_layers outside 1..8, a
 * null table or layer pointer, or overlapping outputs, and ALIGNMENT for
 * the stride.
 */
dbf_status dbf_forward_grouped(const void* x, int64_t ldx, int64_t T, int32_t num_layers,
                               const uint32_t* const* B1s, const uint32_t* const* B2s,
                               const void* const* alphas, const void* const* betas,
                               const void* const* gammas, int64_t N, int64_t R, int64_t M,
                               int32_t ell, void* y, int64_t ldy, int64_t y_layer_stride,
                               dbf_dtype y_type, uint32_t flags, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Workspace bytes needed by dbf_backward for these sizes.
 * Errors: INVALID_ARG if N, R, M <= 0 (or above DBF_MAX_DIM), ell < 1,
 * T <= 0 or bytes == NULL.
 */
dbf_status dbf_backward_workspace_bytes(int64_t N, int64_t R, int64_t M, int32_t ell, int64_t T,
                                        size_t* bytes);

/*
 * Backward pass of one layer for quantisation-aware training (LoRDBA
 * summary, section 2, "Pipeline de Entrenamiento", steps 3-4: the sign
 * carriers B = sign(H) and the scale vectors are trained together; the
 * gradient passes sign() through a soft-sign straight-through estimator
 * with a temperature).  With g = dL/dy [T][N] for y = dbf_forward(x), per
 * term i: V_i = x.gamma_i, U_i = V_i B2^T, Z_i = U_i.beta_i,
 * W_i = Z_i B1^T, P_i = (g.alpha_i) B1, Q_i = (P_i.beta_i) B2; then
 *   dalpha_i[n] = sum_t g[t][n] W_i[t][n]     dalpha [ell][N] fp32
 *   dbeta_i[r]  = sum_t U_i[t][r] P_i[t][r]   dbeta  [ell][R] fp32
 *   dgamma_i[m] = sum_t x[t][m] Q_i[t][m]     dgamma [ell][M] fp32
 *   dx = sum_i Q_i.gamma_i                    dx [T][lddx], dx_type F16|F32
 *   dS1 = sum_i (g.alpha_i)^T Z_i             [N][R] fp32, row-major, or NULL
 *   dS2 = sum_i (P_i.beta_i)^T V_i            [R][M] fp32, row-major, or NULL
 *   dH1 = dS1 * (1 - tanh(H1/tau)^2) / tau    with latents H1 [N][R], H2
 *   dH2 = dS2 * (1 - tanh(H2/tau)^2) / tau    [R][M] (fp32, row-major)
 * (reading of the estimator: the soft sign is tanh(h/tau); tau > 0 is the
 * caller's current temperature).  H1 and dH1 are both given or both NULL,
 * likewise H2 and dH2; dS1/dS2 may be NULL whether or not dH is wanted.
 *   x [T][ldx], g [T][ldg] fp16; B1, B2 packed as for dbf_forward; B1t and
 *   B2t the packed transposes (dbf_transpose_signs of B1 as N x R, of B2 as
 *   R x M); alpha, beta, gamma [ell][*] fp16.
 * Precision: fp32 accumulation; every matrix-core operand (V, g.alpha, Z,
 * P.beta) is rounded to fp16 once.  Outputs are written, not accumulated.
 * All device memory is the caller's; work is asynchronous on `stream`.
 * Alignment: x, g, B1, B2, B1t, B2t and ws 16-byte aligned; ldx and ldg
 * multiples of 8; fp32 outputs and latents 4-byte aligned.
 * Errors: INVALID_ARG (null required pointer, sizes <= 0 or above
 * DBF_MAX_DIM, ell * T too large, ld below the width, unpaired H/dH, tau
 * not positive and finite, bad dtype), ALIGNMENT, WORKSPACE (ws_bytes below
 * dbf_backward_workspace_bytes), HIP.
 */
dbf_status dbf_backward(const void* x, int64_t ldx, const void* g, int64_t ldg, const uint32_t* B1,
                        const uint32_t* B2, const uint32_t* B1t, const uint32_t* B2t,
                        const void* alpha, const void* beta, const void* gamma, int64_t N,
                        int64_t R, int64_t M, int32_t ell, int64_t T, void* dx, int64_t lddx,
                        dbf_dtype dx_type, float* dalpha, float* dbeta, float* dgamma, float* dS1,
                        float* dS2, const float* H1, const float* H2, float tau, float* dH1,
                        float* dH2, void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace bytes needed by dbf_factorize for an N x M matrix and inner
 * dimension k.  Errors: INVALID_ARG for sizes <= 0 or above DBF_MAX_DIM, or
 * bytes == NULL.
 */
dbf_status dbf_factorize_workspace_bytes(int64_t N, int64_t M, int64_t k, size_t* bytes);

/*
 * Double binary factorisation of a dense matrix (DBF summary, section 2,
 * "Algoritmo de Optimizacion"): W ~ (diag(alpha) S1 diag(beta)) (S2
 * diag(gamma)), S1 [N][k] and S2 [k][M] sign matrices, so that dbf_forward
 * with these factors (ell = 1, after dbf_pack_signs) applies the
 * approximation of W.  Alternating minimisation over the two factors; each
 * half step runs admm_iters ADMM iterations (scaled form, penalty rho0 *
 * trace(Gram) / k) that project onto scaled sign matrices with SVID (sign
 * times the rank-1 approximation of the magnitude, here by power_iters power
 * steps warm-started across iterations; the linear solves by Newton-Schulz
 * inversion of the k x k regularised Gram matrix).  outer alternations (0:
 * only the start is projected).
 *   W      fp32 [N][ldw] (ldw >= M)
 *   omega  fp32 [k][N] Gaussian sketch drawn by the caller: the start is
 *          Y0 = SVID(omega W); or NULL with
 *   X0, Y0 fp32 [N][k], [k][M] scaled sign matrices to start from (both or
 *          neither)
 *   S1, S2 int8 +-1 outputs [N][k], [k][M]; alpha [N], beta [k], gamma [M]
 *          fp16 outputs; rel_err: device fp32 scalar ||W - W~||_F / ||W||_F,
 *          or NULL.
 * Reading of the method where the page is silent: the row scale of the
 * second factor is folded into beta; the first factor starts from SVID of
 * the regularised least-squares solution.  All arithmetic is fp32.
 * Errors: INVALID_ARG (null output, neither omega nor a start, sizes, ldw <
 * M, outer < 0, admm_iters or power_iters < 1, rho0 not positive and
 * finite), ALIGNMENT (fp32 inputs 4-byte, fp16 outputs 2-byte, ws 16-byte),
 * WORKSPACE, HIP.
 */
dbf_status dbf_factorize(const float* W, int64_t N, int64_t M, int64_t ldw, int64_t k,
                         const float* omega, const float* X0, const float* Y0, int32_t outer,
                         int32_t admm_iters, int32_t power_iters, float rho0, int8_t* S1,
                         int8_t* S2, void* alpha, void* beta, void* gamma, float* rel_err,
                         void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DBF_H_ */
