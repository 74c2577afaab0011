// Large-T (prefill) stages of one adapter as token tiles shared through LDS.
//
// Each stage is a dense contraction once the signs are +-1 (DBF summary,
// section 2, inference: the product with the weight becomes two products
// with sign matrices), run on v_mfma_f32_16x16x32_f16 with fp32
// accumulation:
//   stage 1:  z_i[t][r] = fp16(beta_i[r] * sum_m S2[r][m] * fp16(gamma_i[m] * x[t][m]))
//   stage 2:  y[t][n]   = sum_i alpha_i[n] * sum_r S1[n][r] * z_i[t][r]
// z lives in the workspace as fp16 rows [ell][T][ldz] (ldz = R rounded up
// to 8).
//
// A workgroup owns W row quads (64 output rows each) x 16*NC tokens and
// runs KS*W waves: wave (wq, kp) computes quad wq of the workgroup over the
// 128-blocks kb = KS*j + kp of the reduction.  Per iteration j the
// workgroup stages the token operand of its KS blocks (16*NC token rows x
// 256 bytes each), every wave's sign words and (stage 1) gamma from global
// memory straight into LDS with global_load_lds, and every wave of the
// same K-part reads the token tile as its MFMA B operand, so each staged
// byte feeds W row quads.  Stage 1 multiplies the staged x by gamma_i
// before the MFMA (one fp16 rounding of the exact product, as the separate
// prep kernel of the multi-adapter path does).
//
// Sign expansion: for step s of a block, ((w << (3-s)) & 0x88888888) |
// 0x22222222 holds the lane's 8 signs of that step as e2m1 +-1.0 (the
// packed bit order puts slot 8s+e at bit 4e+s), and four
// v_cvt_scalef32_pk_f16_fp4 turn its bytes into the four f16 pairs of the A
// operand: 6 VALU ops per 16x32 operand, each feeding NC MFMAs.
//
// The LDS holds NBUF pipeline buffers with NBUF-1 iterations' requests in
// flight and one barrier per iteration; each wave spreads its requests for
// a later iteration over the steps of the current one.  The K-parts'
// partial tiles are summed in a fixed order through LDS at the end, so
// results do not depend on timing.
#include <climits>

#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

namespace {

typedef const DBF_GLOBAL v8h* gv8hp;
typedef const DBF_GLOBAL uint16_t* gu16p;

constexpr int64_t kComputeUnitsTile = 256;  // MI355X

struct TileParams {
  const uint32_t* S;  // packed signs, rows x K
  const half_t* b;    // token operand rows [T][ldb]: x (stage 1) or z_0 (stage 2)
  int64_t ldb;
  int64_t b_term;     // halfs between the terms' operands (stage 2; 0 in stage 1)
  const half_t* gam;  // stage 1: gamma [ell][K]
  const half_t* scl;  // stage 1: beta [ell][rows]; stage 2: alpha [ell][rows]
  void* out;          // stage 1: z [ell][T][ldo] fp16; stage 2: y [T][ldo]
  int64_t ldo;
  int64_t o_term;     // stage 1: halfs between the terms' z
  int32_t rows, K, T, ell, nkb, nq;
  int32_t n_rg, n_tb, grid;
  int32_t remap;      // 1: workgroup b takes item (b%8)*(grid/8) + b/8 (consecutive items per XCD)
  int32_t tb_major;   // 1: items ordered token block first, else row group first
  int32_t y_f32, accumulate;
  uint32_t nib_mask, nib_one;  // 0x88888888, 0x22222222 (kept in registers)
};

// f(integral_constant<int, I>) for I = B .. E-1 in order.
template <int B, int E, class F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int STAGE, int NC, int W, int KS, int NBUF>
struct TileShape {
  static constexpr int NWV = W * KS;                 // waves
  static constexpr int NT = 64 * NWV;                // threads
  static constexpr int ROWS = 16 * NC;               // tokens per workgroup
  static constexpr int TILE = ROWS * 256;            // bytes of one staged 128-block
  static constexpr int JB = ROWS / (4 * W);          // 1 KB token blocks a wave loads per iteration
  static constexpr int SGN = NWV * 1024;             // every wave's sign words
  static constexpr int GAM = STAGE == 1 ? KS * 256 : 0;  // gamma of each K-part's block
  static constexpr int BUF = KS * TILE + SGN + GAM;  // one pipeline buffer
  // requests per wave per iteration: JB token blocks and the sign words,
  // plus (stage 1) the gamma block for the waves of quad 0 of the
  // workgroup
  static constexpr int GROUP = JB + 1 + (STAGE == 1 ? 1 : 0);
  static constexpr int GROUP_NQ0 = JB + 1;
  static constexpr int TPW = 4 * NC / KS;            // output tiles each wave finishes
  static constexpr int RED = KS * W * 4 * NC * 64 * 16;  // every wave's partial tiles
  static constexpr int BYTES = NBUF * BUF > RED ? NBUF * BUF : RED;
  static_assert(ROWS % (4 * W) == 0 && JB * NWV * 4 == KS * ROWS, "token blocks per wave");
  static_assert(TPW * KS == 4 * NC, "tiles per wave");
  static_assert(NBUF >= 2 && (NBUF - 2) * GROUP < 64, "pipeline depth");
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// NBUF buffers for shape (NC, W, KS): as many as fit in the LDS, at most 6.
template <int STAGE, int NC, int W, int KS>
constexpr int tile_nbuf() {
  constexpr int b = TileShape<STAGE, NC, W, KS, 2>::BUF;
  constexpr int n = (159 * 1024) / b;
  return n > 6 ? 6 : (n < 2 ? 2 : n);
}

template <int STAGE, int NC, int W, int KS, int NBUF, bool ELL1>
__global__ __launch_bounds__(64 * W * KS) void k_tile(TileParams p) {
  typedef TileShape<STAGE, NC, W, KS, NBUF> Sh;
  __shared__ __attribute__((aligned(1024))) char lds[Sh::BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wv % W, kp = wv / W;
  const int g = lane >> 4, c16 = lane & 15;

  const int b = blockIdx.x;
  const int item = p.remap ? (b & 7) * (p.grid >> 3) + (b >> 3) : b;
  int tb, rg;
  if (p.tb_major) {
    tb = item / p.n_rg;
    rg = item - tb * p.n_rg;
  } else {
    rg = item / p.n_tb;
    tb = item - rg * p.n_tb;
  }
  const int q = rg * W + wq;
  const bool qok = q < p.nq;
  const int t0 = tb * Sh::ROWS;
  const int nkb = p.nkb, K = p.K, T = p.T;
  const int niter = (nkb + KS - 1) / KS;
  const int last = niter - 1;
  // iterations whose KS blocks are whole (no clamping of the reduction index)
  const int nwhole = K / (KS * kColBlock);
  // first entry of the last whole 8-entry chunk of a row: x rows hold M
  // entries (a multiple of 8), z rows ldz (zero-padded past R)
  const int kmax = (STAGE == 1 ? K : (int)p.ldb) - 8;

  // Token block j of this wave (1 KB of LDS, token rows 4u..4u+3 of
  // K-part kpb): lane L loads 16-byte chunk (L%16) ^ (row%16) of row
  // 4u + L/16, so the chunk of row r at column c lands at LDS position
  // c ^ (r % 16) of the row, and the operand reads below hit distinct banks.
  // Rows past T repeat row T-1 (their output columns are never stored).
  // Byte offsets of a row are 32-bit (the host checks T * ldb * 2 < 2^31).
  uint32_t roff[Sh::JB];
  int rkp[Sh::JB];
#pragma unroll
  for (int j = 0; j < Sh::JB; ++j) {
    const int blk = wv + j * Sh::NWV;
    rkp[j] = blk / (Sh::ROWS / 4);
    const int row = (blk % (Sh::ROWS / 4)) * 4 + (lane >> 4);
    const int t = t0 + row < T ? t0 + row : T - 1;
    roff[j] = (uint32_t)t * (uint32_t)p.ldb * 2u + (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
  }
  const char* sq = (const char*)p.S + ((int64_t)(qok ? q : 0) * nkb << 10);

  float ys[ELL1 ? 1 : Sh::TPW][1][4];  // stage 2 with several terms: running sum

  for (int i = 0; i < (ELL1 ? 1 : p.ell); ++i) {
    const char* bterm = (const char*)p.b + (int64_t)i * p.b_term * 2;
    const char* gami = STAGE == 1 ? (const char*)(p.gam + (int64_t)i * K) : nullptr;
    // this wave's row scales (lane L: row 64q + L), kept as loaded
    const int srow_s = q * 64 + lane;
    const half_t sclh = p.scl[(int64_t)i * p.rows + (srow_s < p.rows ? srow_s : p.rows - 1)];

    // Request j of iteration it into pipeline buffer bf: this wave's token
    // blocks (j < JB), its sign words (j = JB) and (stage 1, by the waves
    // of quad 0) its K-part's 128 entries of gamma (j = JB + 1).
    // Iterations past the last repeat the last one's addresses.
    auto issue_part = [&](int it, int bf, auto jc) {
      constexpr int j = decltype(jc)::value;
      it = it < last ? it : last;
      const uint32_t lb = lds0 + bf * Sh::BUF;
      if constexpr (j < Sh::JB) {
        const int blk = wv + j * Sh::NWV;
        if (it < nwhole) {
          dma16(bterm, roff[j] + (uint32_t)(it * KS + rkp[j]) * 256u, lb + blk * 1024);
        } else {
          // chunk column of this lane and its first entry, clamped
          const int row = (blk % (Sh::ROWS / 4)) * 4 + (lane >> 4);
          const int c = (lane & 15) ^ (row & 15);
          int k = (it * KS + rkp[j]) * kColBlock + 8 * c;
          k = k < kmax ? k : kmax;
          dma16(bterm, roff[j] - (uint32_t)(c * 16) + (uint32_t)k * 2u, lb + blk * 1024);
        }
      } else if constexpr (j == Sh::JB) {
        int kb = it * KS + kp;
        kb = kb < nkb ? kb : nkb - 1;
        dma16(sq, (uint32_t)((kb << 10) + lane * 16), lb + KS * Sh::TILE + wv * 1024);
      } else if constexpr (STAGE == 1) {
        if (wq == 0) {  // lane L: entries 2L, 2L+1 of K-part kp's block
          int k = (it * KS + kp) * kColBlock + 2 * lane;
          k = k < K - 2 ? k : K - 2;
          dma4(gami, (uint32_t)k * 2u, lb + KS * Sh::TILE + Sh::SGN + kp * 256);
        }
      }
    };
    // the requests j of iteration it with first <= j < last (in order)
    auto issue_range = [&](int it, int bf, auto firstc, auto lastc) {
      static_for<decltype(firstc)::value, decltype(lastc)::value>(
          [&](auto jc) { issue_part(it, bf, jc); });
    };
    auto issue = [&](int it, int bf) {
      issue_range(it, bf, std::integral_constant<int, 0>{},
                  std::integral_constant<int, Sh::GROUP>{});
    };

    v4f acc[4][NC];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[h][c] = v4f{0.f, 0.f, 0.f, 0.f};

    // One step's token operands (each token tile's v8h) and, in stage 1,
    // its gamma entries, read from pipeline buffer bf.
    struct StepOps {
      v8h bv[NC];
      v8h gv;
    };
    auto load_step = [&](int bf, int s, StepOps& o) {
      const char* bb = lds + bf * Sh::BUF;
      const char* bl = bb + kp * Sh::TILE;
      if constexpr (STAGE == 1)
        o.gv = *(const v8h*)(bb + KS * Sh::TILE + Sh::SGN + kp * 256 + (4 * s + g) * 16);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        o.bv[c] = *(const v8h*)(bl + (16 * c + c16) * 256 + (((4 * s + g) ^ c16) << 4));
    };
    // Which of the requests of the next group a step issues: with three or
    // more buffers a quarter per step (issued together right after the
    // barrier, the workgroup's requests queue at the texture unit and hold
    // up every wave's MFMAs); with two, all at the first step (the group is
    // waited for at the next iteration).
    auto req_lo = [](int s) { return NBUF > 2 ? s * Sh::GROUP / 4 : (s == 0 ? 0 : Sh::GROUP); };

    // Iteration it: the MFMAs of its KS blocks from buffer it % NBUF.  Each
    // step reads the next step's operands ahead of its own MFMAs and then
    // issues its share of the requests of iteration it + NBUF - 1 into
    // buffer (it - 1) % NBUF, which every wave finished reading in
    // iteration it - 1.  PART: a block of it may be the reduction's partial
    // last one or lie past it (its entries from K on contribute zero).
    auto body = [&](int it, auto part_c) {
      constexpr bool PART = decltype(part_c)::value;
      // this wave's requests of it done (requests complete in issue order;
      // the bound is exact per wave), then every wave's
      if (wq == 0)
        wait_vm_lds<(NBUF - 2) * Sh::GROUP>();
      else
        wait_vm_lds<(NBUF - 2) * Sh::GROUP_NQ0>();
      __syncthreads();
      const int bf = it % NBUF, rbf = (it + NBUF - 1) % NBUF;
      const v4u w = *(const v4u*)(lds + bf * Sh::BUF + KS * Sh::TILE + wv * 1024 + lane * 16);
      const int kvalid = K - (it * KS + kp) * kColBlock;
      StepOps ops[2];
      load_step(bf, 0, ops[0]);
      auto step = [&](auto scst) {
        constexpr int s = decltype(scst)::value;
        if constexpr (s < 3) load_step(bf, s + 1, ops[(s + 1) & 1]);
        const StepOps& o = ops[s & 1];
        v8h a[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) a[h] = expand_cvt<s>(w[h], p.nib_mask, p.nib_one);
        const bool live = !PART || 32 * s + 8 * g < kvalid;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          v8h b = o.bv[c];
          if constexpr (STAGE == 1) b = b * o.gv;
          if constexpr (PART) {
            if (!live) b = v8h{};
          }
#pragma unroll
          for (int h = 0; h < 4; ++h)
            acc[h][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[h], b, acc[h][c], 0, 0, 0);
        }
        static_for<req_lo(s), req_lo(s + 1)>(
            [&](auto jc) { issue_part(it + NBUF - 1, rbf, jc); });
        // keep each step's reads, MFMAs and requests together (the
        // scheduler would sink every read next to its use)
        __builtin_amdgcn_sched_barrier(0);
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
    };

    // Pipeline over NBUF buffers with the requests of NBUF - 1 iterations
    // in flight.
    if (i > 0) __syncthreads();  // the previous term's readers of lds are done
#pragma unroll
    for (int d = 0; d < NBUF - 1; ++d) issue(d, d);
    // The loop holds no branch around the MFMAs (a branch there makes the
    // compiler copy the accumulators every iteration): iterations whose KS
    // blocks are all present and whole run first; the last one, when its
    // blocks are partial or missing, runs masked.  Waves of a quad past the
    // last one compute on quad 0's signs and store nothing.
    const int nmain = K % kColBlock == 0 ? nkb / KS : (nkb - 1) / KS;
    int it = 0;
    for (; it < nmain; ++it) body(it, std::false_type{});
    if (it < niter) body(it, std::true_type{});
    wait_vm<0>();
    __syncthreads();

    // The K-parts' partial tiles are summed in a fixed order (part 0 first)
    // through LDS, which every request has filled and every wave has
    // finished reading; wave (wq, kp) then finishes tiles kp*TPW .. of its
    // quad, so the epilogue is spread over the K-parts' waves.
    float tsum[Sh::TPW][4];
    if constexpr (KS > 1) {
      v4f* red = (v4f*)lds;
      auto slot = [&](int part, int tile) { return ((part * W + wq) * 4 * NC + tile) * 64 + lane; };
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < NC; ++c) red[slot(kp, h * NC + c)] = acc[h][c];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < Sh::TPW; ++e) {
        v4f sum = red[slot(0, kp * Sh::TPW + e)];
#pragma unroll
        for (int part = 1; part < KS; ++part) sum += red[slot(part, kp * Sh::TPW + e)];
#pragma unroll
        for (int v = 0; v < 4; ++v) tsum[e][v] = sum[v];
      }
    } else {
#pragma unroll
      for (int e = 0; e < Sh::TPW; ++e)
#pragma unroll
        for (int v = 0; v < 4; ++v) tsum[e][v] = acc[e / NC][e % NC][v];
    }

    if (qok) {
      const float scl_l = srow_s < p.rows ? (float)sclh : 0.0f;
      const int nterm = ELL1 ? 1 : p.ell;
#pragma unroll
      for (int e = 0; e < Sh::TPW; ++e) {
        const int tile = kp * Sh::TPW + e, h = tile / NC, c = tile % NC;
        const int rl = h * kRowTile + 4 * g;  // quad-local row of v = 0
        float sv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[v] = __shfl(scl_l, rl + v, 64);
        const int r0 = q * 64 + rl;
        const int t = t0 + 16 * c + c16;
        if (STAGE == 1) {
          if (t < T) {
            half_t* zp = (half_t*)p.out + (int64_t)i * p.o_term + (int64_t)t * p.ldo + r0;
            const v4h zv = v4h{(half_t)(tsum[e][0] * sv[0]), (half_t)(tsum[e][1] * sv[1]),
                               (half_t)(tsum[e][2] * sv[2]), (half_t)(tsum[e][3] * sv[3])};
            // z rows are zero-padded from R up to ldz (a multiple of 8), so
            // stage 2 reads whole chunks
            if (r0 + 4 <= p.rows) {
              *(v4h*)zp = zv;
            } else if (r0 < p.ldo) {
              v4h zz = zv;
              for (int v = 0; v < 4; ++v)
                if (r0 + v >= p.rows) zz[v] = (half_t)0.0f;
              *(v4h*)zp = zz;
            }
          }
        } else {
          float o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float term = tsum[e][v] * sv[v];
            if constexpr (ELL1) {
              o[v] = term;
            } else {
              ys[e][0][v] = i == 0 ? term : ys[e][0][v] + term;
              o[v] = ys[e][0][v];
            }
          }
          if (i + 1 == nterm && t < T && r0 < p.rows) {
            if (p.accumulate) {
              float old[4];
              load4(p.out, p.ldo, p.y_f32, t, r0, p.rows, old);
#pragma unroll
              for (int v = 0; v < 4; ++v) o[v] += old[v];
            }
            store4(p.out, p.ldo, p.y_f32, t, r0, p.rows, o);
          }
        }
      }
    }
  }
}

// Tile shapes compiled: (NC, W, KS), 8 waves per workgroup (two per SIMD:
// with one, a wave's sign expansion and MFMAs barely overlap).
struct TileChoice {
  int nc, w, ks;
};
constexpr TileChoice kTileChoices[] = {{4, 4, 2}, {4, 2, 4}, {2, 2, 4}, {2, 1, 8}};

template <int NC, int W, int KS>
constexpr int tile_bytes() {
  return TileShape<1, NC, W, KS, tile_nbuf<1, NC, W, KS>()>::BYTES;
}
int lds_of(const TileChoice& c) {
  if (c.nc == 4 && c.w == 4) return tile_bytes<4, 4, 2>();
  if (c.nc == 4 && c.w == 2) return tile_bytes<4, 2, 4>();
  if (c.nc == 2 && c.w == 2) return tile_bytes<2, 2, 4>();
  return tile_bytes<2, 1, 8>();
}

// Estimated cycles of one stage for a tile shape: per iteration the larger
// of the MFMA time of a SIMD (its two waves' 16*NC MFMAs each, at the
// issue rate measured with the expansion in the loop) and the LDS fill at
// about 46 bytes per cycle and compute unit (measured); a fixed cost per
// workgroup (argument loads, first requests, stores) plus the sum of its
// KS K-parts; and rounds when there are more workgroups than fit at once.
double tile_cost(const TileChoice& c, int64_t nq, int64_t nkb, int64_t T) {
  const int64_t n_rg = cdiv(nq, c.w), n_tb = cdiv(T, 16 * c.nc);
  const int64_t wgs = n_rg * n_tb;
  const int slots = (160 * 1024) / lds_of(c);
  const int64_t rounds = cdiv(wgs, kComputeUnitsTile * (slots > 0 ? slots : 1));
  const double cpm = c.nc == 4 ? 19.5 : 25.0;
  const double mfma = 2.0 * 16 * c.nc * cpm;
  const double fill = (c.ks * 16.0 * c.nc * 256 + 8 * 1024 + c.ks * 256) / 46.0;
  const double iter = mfma > fill ? mfma : fill;
  return rounds * (cdiv(nkb, c.ks) * iter + 4600.0 + 600.0 * c.ks);
}

template <int STAGE, int NC, int W, int KS>
hipError_t launch_tile_k(TileParams p, hipStream_t s) {
  typedef TileShape<STAGE, NC, W, KS, 2> Sh;
  p.n_rg = (int32_t)cdiv(p.nq, W);
  p.n_tb = (int32_t)cdiv(p.T, Sh::ROWS);
  const int64_t grid = (int64_t)p.n_rg * p.n_tb;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  p.grid = (int32_t)grid;
  p.remap = grid % 8 == 0 ? 1 : 0;
  constexpr int NB = tile_nbuf<STAGE, NC, W, KS>();
  if (p.ell == 1)
    hipLaunchKernelGGL((k_tile<STAGE, NC, W, KS, NB, true>), dim3((unsigned)grid), dim3(Sh::NT), 0,
                       s, p);
  else
    hipLaunchKernelGGL((k_tile<STAGE, NC, W, KS, NB, false>), dim3((unsigned)grid), dim3(Sh::NT),
                       0, s, p);
  return hipGetLastError();
}

template <int STAGE>
hipError_t launch_tile_stage(TileParams p, hipStream_t s) {
  p.nq = (int32_t)cdiv(p.rows, kRowTile * kQuad);
  p.nkb = (int32_t)cdiv(p.K, kColBlock);
  const TileChoice* best = &kTileChoices[0];
  double best_cost = 1e300;
  for (const TileChoice& c : kTileChoices) {
    const double cost = tile_cost(c, p.nq, p.nkb, p.T);
    if (cost < best_cost) {
      best_cost = cost;
      best = &c;
    }
  }
  // replicate in the XCDs' L2s whichever operand is smaller: items ordered
  // token block first share the token operand within an XCD and read every
  // sign unit once per XCD, and conversely
  const int64_t sign_bytes = (int64_t)p.nq * p.nkb * 1024;
  const int64_t tok_bytes = (int64_t)p.T * p.nkb * 256;
  p.tb_major = sign_bytes <= tok_bytes ? 1 : 0;
  const TileChoice c = *best;
  if (c.nc == 4 && c.w == 4) return launch_tile_k<STAGE, 4, 4, 2>(p, s);
  if (c.nc == 4 && c.w == 2) return launch_tile_k<STAGE, 4, 2, 4>(p, s);
  if (c.nc == 2 && c.w == 2) return launch_tile_k<STAGE, 2, 2, 4>(p, s);
  return launch_tile_k<STAGE, 2, 1, 8>(p, s);
}

}  // namespace

// Whether the token-tile stages take this call: the staging addresses its
// token operand rows with 32-bit byte offsets.
bool tile_path_fits(const ForwardArgs& a) {
  const int64_t lim = (int64_t)1 << 31;
  bool ok = a.M % 8 == 0 && a.T * a.ldx * 2 + a.M * 2 < lim &&
            a.T * ldz_of(a.R) * 2 + a.R * 2 < lim;
  // gamma is read in 16-byte chunks
  for (int j = 0; j < (a.group > 1 ? a.group : 1); ++j)
    ok = ok && (((uintptr_t)(a.group > 1 ? a.grp[j].gamma : a.single.gamma)) & 15u) == 0;
  return ok;
}

// The two stages of one adapter with the shared token tiles (one launch
// each).  The caller has validated the arguments and tile_path_fits.
hipError_t launch_tile_forward(const ForwardArgs& a, hipStream_t s) {
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  half_t* z = (half_t*)((char*)a.ws + L.z);
  const int64_t ldz = ldz_of(a.R);
  TileParams p{};
  p.T = (int32_t)a.T;
  p.ell = a.ell;
  p.nib_mask = 0x88888888u;
  p.nib_one = 0x22222222u;
  if (a.phases & 2) {
    TileParams p1 = p;
    p1.S = a.single.B2;
    p1.b = a.x;
    p1.ldb = a.ldx;
    p1.b_term = 0;
    p1.gam = a.single.gamma;
    p1.scl = a.single.beta;
    p1.out = z;
    p1.ldo = ldz;
    p1.o_term = a.T * ldz;
    p1.rows = (int32_t)a.R;
    p1.K = (int32_t)a.M;
    const hipError_t e = launch_tile_stage<1>(p1, s);
    if (e != hipSuccess) return e;
  }
  if (a.phases & 4) {
    TileParams p2 = p;
    p2.S = a.single.B1;
    p2.b = z;
    p2.ldb = ldz;
    p2.b_term = a.T * ldz;
    p2.scl = a.single.alpha;
    p2.out = a.y;
    p2.ldo = a.ldy;
    p2.rows = (int32_t)a.N;
    p2.K = (int32_t)a.R;
    p2.y_f32 = a.y_f32;
    p2.accumulate = a.accumulate;
    return launch_tile_stage<2>(p2, s);
  }
  return hipSuccess;
}

}  // namespace dbf
