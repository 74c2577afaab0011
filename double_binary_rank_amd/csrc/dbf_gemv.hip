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
// Launches: prep(x) (with several adapters one extra workgroup also builds
// the column blocks) -> stage 1 (writes z = beta*u, fp32) -> prep(z) ->
// stage 2.
#include <climits>

#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

// ------------------------------------------------------------ fp8 parts ----

__device__ inline int floor_log2_pos(float m) {
  return (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127;
}

// fp8 parts use the hardware conversion v_cvt_pk_fp8_f32: OCP e4m3 (3
// mantissa bits, subnormal step 2^-9), round to nearest even, for the
// scaled values |a| < 256 given here; v_cvt_f32_fp8 decodes a code exactly.
// On gfx950 it agrees, code and value, with the direct definition (round
// m / 2^(e-3), or m * 512 below 2^-6, to an integer, nearest even) on every
// 2^-12 step of [-256, 256), which holds every tie, and on 8M random fp32
// values.

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
  // multi-adapter column blocks, built by the extra workgroup 0 (none when
  // seg_cbl is null)
  ColBlock* seg_cbl;
  WsHeader* seg_hdr;
  int32_t seg_chunk;
};

// K order of an fp8 operand of v_mfma_scale_f32_16x16x128_f8f6f4 inside a
// 128-block: lane group g holds bytes e = 0..15 for k = 16g + e and bytes
// e = 16..31 for k = 64 + 16g + (e - 16).  (The fp4 operand holds 32
// consecutive k = 32g + e; measured on gfx950 with one-hot operands.)
// Byte offset of the operand's k-th entry inside one part's 128 bytes:
__device__ inline int fp8_operand_byte(int k) {
  const int h = k >> 6, r = k & 63;           // half, position in the half
  return (r >> 4) * 32 + h * 16 + (r & 15);   // lane group (r/16), byte e
}

// The fp4 operand's k-th entry (lane group k/32, slot k%32) carries the sign
// of block col slot_col(k/32, k%32); the inverse swaps the same two 2-bit
// fields of the col index, so col c meets operand entry
__device__ inline int operand_k_of_col(int c) {
  return ((c & 0x18) << 2) | ((c & 0x60) >> 2) | (c & 7);
}

// Maximum over the wave, returned in every lane: DPP within rows of 16
// (quad swaps, then half-row and row mirrors), then the four row maxima
// read as scalars; no LDS traffic.
template <int ctrl>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The kParts fp8 parts of one 128-block whose entries 2*lane and 2*lane+1
// this lane holds; every lane of the wave must call it (wave reductions).
// Each part has one E8M0 scale for the whole block (the block maximum is a
// wave reduction), so the scale is the same whichever 32 entries the
// hardware attaches a lane's scale to.  For each part, put(part, code, s)
// receives the pair's e4m3 codes (entry 2*lane in the low byte) and the
// part's scale exponent s; the pair's byte offset inside the part's 128
// operand bytes is fp8_operand_byte(operand_k_of_col(2*lane)).
template <typename Put>
__device__ inline void block_parts(float v0, float v1, Put&& put) {
#pragma unroll
  for (int part = 0; part < kParts; ++part) {
    const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    int s = mx > 0.0f ? floor_log2_pos(mx) - 7 : 0;  // scaled block max in [128, 256)
    s = s < -127 ? -127 : (s > 127 ? 127 : s);
    const float down = __builtin_ldexpf(1.0f, -s), up = __builtin_ldexpf(1.0f, s);
    const int codes = __builtin_amdgcn_cvt_pk_fp8_f32(v0 * down, v1 * down, 0, false);
    const float q0 = __builtin_amdgcn_cvt_f32_fp8(codes, 0), q1 = __builtin_amdgcn_cvt_f32_fp8(codes, 1);
    v0 -= q0 * up;  // exact: q*up is v rounded on a grid no finer than v's own
    v1 -= q1 * up;
    put(part, (uint16_t)codes, s);
  }
}

// One wave per (term, token, 128-block); lane l owns entries 2l and 2l+1.
template <bool MULTI>
__global__ __launch_bounds__(256) void k_prep(PrepParams p) {
  if (MULTI && p.seg_cbl != nullptr && blockIdx.x == 0) {
    segment_ids(p.ids, (int32_t)p.T, p.num_adapters, p.seg_chunk, p.seg_cbl, p.seg_hdr);
    return;
  }
  const int lane = threadIdx.x & 63;
  // block counts fit 32 bits (the workspace bounds them; the host checks)
  const int blk = ((int)blockIdx.x - (MULTI && p.seg_cbl != nullptr ? 1 : 0)) * 4 + (threadIdx.x >> 6);
  const int nkb = (int)p.nkb, T = (int)p.T;
  if (blk >= p.ell * T * nkb) return;  // uniform per wave
  const int r = blk / nkb, kb = blk - r * nkb;
  const int i = r / T, t = r - i * T;
  const int kl = 2 * lane;
  const int64_t k = (int64_t)kb * kColBlock + kl;

  bool live = true;
  const half_t* gam = p.gamma;
  if (MULTI) {
    const int32_t ad = p.ids[t];
    live = ad >= 0 && ad < p.num_adapters;
    if (live && !p.from_z) gam = p.gammas[ad];
  }
  // entries from addresses clamped into the row, each in a register of its
  // own, range-checked at the use: the requests go out together
  float v0 = 0.0f, v1 = 0.0f;
  if (live) {
    const int64_t k0 = k < p.K ? k : p.K - 1, k1 = k + 1 < p.K ? k + 1 : p.K - 1;
    if (p.from_z) {
      const float* zr = p.z + i * p.zstride + t * p.ldz;
      const float z0 = zr[k0], z1 = zr[k1];
      v0 = k < p.K ? z0 : 0.0f;
      v1 = k + 1 < p.K ? z1 : 0.0f;
    } else {
      typedef const DBF_GLOBAL uint16_t* gu16p;
      const half_t* gi = gam + i * p.K;
      const half_t* xr = p.x + t * p.ldx;
      const uint32_t g0 = *(gu16p)(gi + k0), g1 = *(gu16p)(gi + k1);
      const uint32_t x0 = *(gu16p)(xr + k0), x1 = *(gu16p)(xr + k1);
      auto h = [](uint32_t u) { return (float)__builtin_bit_cast(half_t, (uint16_t)u); };
      v0 = k < p.K ? h(g0) * h(x0) : 0.0f;
      v1 = k + 1 < p.K ? h(g1) * h(x1) : 0.0f;
    }
  }
  uint8_t* out = (uint8_t*)p.opnd + (int64_t)blk * (kParts * 4 * 32);
  // kl even: cols kl, kl+1 meet adjacent operand entries, i.e. adjacent bytes
  const int boff = fp8_operand_byte(operand_k_of_col(kl));
  block_parts(v0, v1, [&](int part, uint16_t code, int s) {
    *(uint16_t*)(out + part * 128 + boff) = code;
    if (lane < 4) p.oscl[(int64_t)blk * (kParts * 4) + part * 4 + lane] = (uint8_t)(s + 127);
  });
}

// ---------------------------------------------------------- stage kernel ----

// 32 sign slots of a packed word as fp4 (e2m1) +-1.0: register d holds slots
// 8d..8d+7, slot 8d+j in nibble j.  Slot 8d+j is stored at bit 4j+d, so a
// left shift by 3-d moves all eight sign bits to the nibble sign positions.
// The constants arrive as kernel arguments (0x88888888, 0x22222222) so that
// they live in registers and each register costs one shift and one and-or.

__device__ inline v8i expand_signs_fp4(uint32_t w, uint32_t msk, uint32_t one) {
  v8i a;
  a[0] = (int)and_or(w << 3, msk, one);
  a[1] = (int)and_or(w << 2, msk, one);
  a[2] = (int)and_or(w << 1, msk, one);
  a[3] = (int)and_or(w, msk, one);
  a[4] = a[5] = a[6] = a[7] = 0;
  return a;
}

struct GemvParams {
  int64_t rows, K, T, nrt, nkb, n_rg;
  int64_t nq, n_qg;      // streaming kernel: row quads, quad groups per column block
  int64_t grid;          // workgroups launched (row-tile kernel)
  int64_t lds_b, lds_s;  // streaming kernel: LDS bytes for staged B operands / their scales
  int32_t ell, tcb;
  uint32_t sign_mask, fp4_one;  // 0x88888888, 0x22222222
  const uint32_t* opnd;
  const uint8_t* oscl;
  const half_t* x;  // stage 1 building its own operand parts: x, stride ldx
  int64_t ldx;
  float* z;
  int64_t ldz, zstride;
  // PIN decode stages: stage 1 splits its reduction into ksplit parts of
  // kslice blocks, part s writing its partial z at z + s * zpart floats;
  // stage 2 adds the ksplit partials (its ZS template argument) in order
  int32_t ksplit, kslice;
  int64_t zpart;
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
  // grouped same-input layers (PIN stages): layer j reads grp[j] and offsets
  // z by j*layer_ws bytes, y by j*y_layer_bytes
  int32_t group;
  int64_t layer_ws, y_layer_bytes;
  Factors grp[kMaxGroup];
};

// Epilogue of one row tile: `sum` is the fp32 MFMA tile of this lane (rows
// 4g..4g+3 of column j).  The kParts parts of a column sit in lanes j, j+1,
// j+2 and are added in that order; stage 1 writes z_i = beta_i * u (fp32),
// stage 2 sums alpha_i * w_i over the ell terms and writes y.  Every lane of
// the wave must call this (it shuffles).
// `srow` gives the per-row output scale of this lane's term (beta_ci for
// stage 1, alpha_ci for stage 2): srow[r] for the rows of `tile`; with
// SCALE_LDS it points into shared memory.
// Value of lane + n within the lane's row of 16 (0 past the row's end):
// DPP row_shl:n, a VALU move with no LDS round trip.
template <int n>
__device__ inline float row_next(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x100 + n, 0xF, 0xF, true));
}

// SCALE: where the row scales come from: 0, srow in device memory; 1, srow
// staged in LDS; 2, the caller's sc_given (the lane's four rows, loaded
// early).
template <int STAGE, int SCALE = 0>
__device__ inline void gemv_epilogue(const GemvParams& p, float* zb, void* yb, const half_t* srow,
                                     v4f sum, int64_t tile, int lane, int g, int part, bool colv,
                                     int ci, int ct, int ntok, int64_t t0,
                                     const half_t* sc_given = nullptr) {
  const int64_t r0 = tile * kRowTile + 4 * g;
  // the parts of a column are lanes j, j+1, j+2 of one row of 16 (j <= 13)
  float tot[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) tot[v] = (sum[v] + row_next<1>(sum[v])) + row_next<2>(sum[v]);
  float sc[4];
  if (SCALE == 2) {
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = (float)sc_given[v];
  } else if (SCALE == 1) {
    // staged rows are zero past p.rows: one 8-byte LDS read, no guards
    typedef const __attribute__((address_space(3))) v4h* lds_v4hp;
    const v4h s4 = *(lds_v4hp)(srow + r0);
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = (float)s4[v];
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) sc[v] = (r0 + v < p.rows) ? (float)srow[r0 + v] : 0.0f;
  }
  if (STAGE == 1) {
    if (part == 0 && colv && r0 < p.rows) {
      float o[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = tot[v] * sc[v];
      store4(zb + ci * p.zstride, p.ldz, true, t0 + ct, r0, p.rows, o);
    }
  } else {
    float val[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) val[v] = (part == 0 && colv) ? tot[v] * sc[v] : 0.0f;
    // sum the ell terms of token ct: their part-0 lanes are 3*(i*ntok + ct);
    // with one term that is this lane itself
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.ell == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] += val[v];
    } else {
      for (int ii = 0; ii < p.ell; ++ii) {
        int src = 16 * g + kParts * (ii * ntok + ct);
        src = src < 64 ? src : lane;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] += __shfl(val[v], src);
      }
    }
    if (part == 0 && colv && ci == 0 && r0 < p.rows) {
      if (p.accumulate) {
        float old[4];
        load4(yb, p.ldy, p.y_f32, t0 + ct, r0, p.rows, old);
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] += old[v];
      }
      store4(yb, p.ldy, p.y_f32, t0 + ct, r0, p.rows, o);
    }
  }
}

// Work item: (column block of <= tcb tokens, group of RTG row tiles).  The
// NW waves split the reduction into interleaved chunks of KC blocks; each
// wave keeps the B operands of its chunk in registers and streams the sign
// blocks of all RTG row tiles against them.  Partial tiles are summed across
// waves in a fixed order through LDS.
// PIN (one adapter, few columns): instead of reading operand parts built by
// a prep launch, each wave requests its sign words, then builds the fp8 parts
// of its own blocks from gamma_i * x (stage 1) or z (stage 2) with the prep
// kernel's arithmetic (block_parts) into its LDS area, so the operands are
// bit for bit those of the two-launch stage.  Every workgroup repeats this
// for its blocks: worth it while a wave's chunk is a few blocks.  Stage 1
// may split its reduction into p.ksplit parts, one work item each, so that
// a short stage fills the compute units: part s writes its partial z (beta
// applied) to its own slice, and stage 2 adds the ZS partials in order as
// it reads z.
constexpr int kPinColTokens = 2;                // PIN: ell * tokens per column block
constexpr int kPinCols = kParts * kPinColTokens;  // PIN: live operand columns

// LDS of one stage: the cross-wave partial tiles, then (PIN) each wave's
// parts, [block][column][128 bytes], and their scale codes (at most kPinCols
// live columns).
template <int RTG, int KC, bool PIN, int NW>
struct GemvLds {
  static constexpr int red_bytes = NW * RTG * 64 * 16;
  static constexpr int pinb_bytes = PIN ? NW * KC * kPinCols * 128 : 16;
  static constexpr int pins_bytes = PIN ? NW * KC * kPinCols : 16;
  static constexpr int bytes = red_bytes + pinb_bytes + pins_bytes;
};

// The work items it = first, first + stride, ... of one stage.
template <int STAGE, int RTG, int KC, bool MULTI, bool PIN, int NW, bool GROUP, int ZS>
__device__ __attribute__((always_inline)) inline void gemv_fp4_items(const GemvParams& p,
                                                                     char* lds, int first,
                                                                     int stride) {
  static_assert(!PIN || !MULTI, "operand parts are built in place for one adapter");
  static_assert(!GROUP || PIN, "grouped layers take the parts-building stages");
  static_assert(!PIN || RTG <= NW, "each wave finishes at most one row tile");
  static_assert(ZS == 1 || (PIN && STAGE == 2), "partial z sums are read by PIN stage 2");
  typedef GemvLds<RTG, KC, PIN, NW> Lds;
  auto red = reinterpret_cast<v4f (*)[RTG][64]>(lds);
  auto pin_b = reinterpret_cast<uint8_t (*)[Lds::pinb_bytes / NW]>(lds + Lds::red_bytes);
  auto pin_s =
      reinterpret_cast<uint8_t (*)[Lds::pins_bytes / NW]>(lds + Lds::red_bytes + Lds::pinb_bytes);
  static_assert(RTG % kQuad == 0, "row tiles come in quads");
  constexpr int RQ = RTG / kQuad;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int c = j / kParts, part = j - kParts * (j / kParts);
  // item counts fit 32 bits (the host checks)
  const int n_cb = MULTI ? p.hdr->n_colblocks : (int)p.n_cb_host;
  // a split stage-1 reduction: the part is the slowest index of an item
  const int nsplit = (STAGE == 1 && PIN && p.ksplit > 1) ? p.ksplit : 1;
  const int n_cbr = n_cb * (int)p.n_rg;
  const int n_per = n_cbr * nsplit;  // items of one layer
  const int n_items = GROUP ? n_per * p.group : n_per;

  for (int it = first; it < n_items; it += stride) {
    int layer = 0, itl = it;
    if constexpr (GROUP) {
      layer = it / n_per;
      itl = it - layer * n_per;
    }
    int ks = 0;
    if constexpr (STAGE == 1 && PIN) {
      ks = itl / n_cbr;
      itl -= ks * n_cbr;
    }
    const int cb = itl / (int)p.n_rg, rg = itl - cb * (int)p.n_rg;
    // the item's reduction blocks [kb_lo, kb_hi) (the host makes every part
    // non-empty)
    const int64_t kb_lo = nsplit > 1 ? (int64_t)ks * p.kslice : 0;
    const int64_t kb_hi =
        nsplit > 1 ? (kb_lo + p.kslice < p.nkb ? kb_lo + p.kslice : p.nkb) : p.nkb;
    float* const zl = (float*)((char*)p.z + (GROUP ? layer * p.layer_ws : 0));
    void* const yl = (char*)p.y + (GROUP ? layer * p.y_layer_bytes : 0);
    int64_t t0, t1;
    int32_t ad;
    Factors f;
    if (MULTI) {
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
      t0 = (int64_t)cb * p.tcb;
      t1 = t0 + p.tcb < p.T ? t0 + p.tcb : p.T;
      ad = 0;
      f = GROUP ? p.grp[layer] : p.single;
    }
    const int64_t tile0 = (int64_t)rg * RTG;
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
    // PIN: wave w < RTG finishes row tile tile0 + w; its row scales are
    // requested now, so the epilogue does not wait for them.  Four 16-bit
    // loads from clamped rows into separate registers, rows past the end
    // zeroed at the use: a select or a packing next to the loads would wait
    // for them here.
    uint32_t scu[4] = {0u, 0u, 0u, 0u};
    int64_t sc_r0 = 0;
    if constexpr (PIN) {
      const int64_t ptile = tile0 + wv < p.nrt ? tile0 + wv : p.nrt - 1;
      const DBF_GLOBAL char* srow = (const DBF_GLOBAL char*)(STAGE == 1 ? f.beta : f.alpha);
      sc_r0 = ptile * kRowTile + 4 * g;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // term ci's row r; rows * ell < 2^31 entries
        const int r = (int)(sc_r0 + v < p.rows ? sc_r0 + v : p.rows - 1) + ci * (int)p.rows;
        scu[v] = *(const DBF_GLOBAL uint16_t*)(srow + 2u * (uint32_t)r);
      }
    }
    const int64_t nrt_here = (p.nrt - tile0) < RTG ? (p.nrt - tile0) : RTG;
    const int nq_here = (int)((nrt_here + kQuad - 1) / kQuad);
    bool first_chunk = true;
    for (int64_t kbase = kb_lo; kbase < kb_hi; kbase += NW * KC) {
      const int64_t kw0 = kbase + wv * KC;
      const int nk = (int)((kb_hi - kw0) < KC ? ((kb_hi - kw0) > 0 ? (kb_hi - kw0) : 0) : KC);
      // lane's 16 bytes of unit (quad, block): the A words of its 4 row tiles
      gv4up base = (gv4up)S + ((tile0 / kQuad) * p.nkb + kw0) * (kUnitWords / 4) + lane;
      v8i bop[KC];
      int bsc[KC];
      v4u wd[RQ][KC];
      auto load_signs = [&]() {
        // every sign word of this round is requested before the first MFMA:
        // RQ*KC 16-byte loads (16 KB per wave at RTG*KC = 64) in flight at
        // once, non-temporal (streamed; measured faster on the decode calls)
#pragma unroll
        for (int rq = 0; rq < RQ; ++rq)
#pragma unroll
          for (int kk = 0; kk < KC; ++kk)
            wd[rq][kk] = (rq < nq_here && kk < nk)
                             ? __builtin_nontemporal_load(base + (rq * p.nkb + kk) * (kUnitWords / 4))
                             : v4u{0u, 0u, 0u, 0u};
      };
      if constexpr (PIN) {
        uint8_t* pb = pin_b[wv];
        uint8_t* ps = pin_s[wv];
        // lane l holds entries 2l, 2l+1 of the block; they meet adjacent
        // operand bytes
        const int boff = fp8_operand_byte(operand_k_of_col(2 * lane));
        // every entry of the wave's blocks is requested before the first
        // part is built (column cc = term * ntok + token, ell * ntok <=
        // kPinColTokens), and the sign words after them: requests return in
        // order, so the parts are built while the signs arrive.
        // Entries k, k+1 (k even) of a row come as one 4-byte word (x, gamma)
        // or 8-byte pair (z), every load from an address inside the row
        // (clamped) and the entries past K zeroed after; columns and blocks
        // the wave does not have are skipped on wave-uniform conditions.  No
        // per-lane branch sits between the requests, so all of them are in
        // flight together.  Stage 1 runs here only with K even and gamma
        // 4-byte aligned (the host checks), so its pairs are aligned words.
        constexpr int NCC = kPinColTokens;
        const int ncc = p.ell * ntok;
        v2f ev[KC][NCC];
        {
          // row starts are wave-uniform; the lane's part is a 32-bit byte
          // offset (a parts-building stage has K <= 256 * 128: at most
          // kMaxZParts parts of at most 32 blocks, or 2 of 64)
          const int kc = STAGE == 1 ? (int)p.K - 2 : (int)p.ldz - 2;
          typedef const DBF_GLOBAL char* gcp;
          uint32_t ea[KC][NCC], eb[KC][NCC];
          v2f ez[ZS][KC][NCC];
#pragma unroll
          for (int kk = 0; kk < KC; ++kk) {
            const int k = (int)(kw0 + kk) * kColBlock + 2 * lane;
            const uint32_t off = (uint32_t)(k < kc ? k : kc) * (STAGE == 1 ? 2u : 4u);
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) {
              const int q = cc / ntok, ci2 = q < p.ell ? q : p.ell - 1;
              const int64_t t = t0 + (cc - q * ntok);
              if (cc >= ncc || kk >= nk) {
                // nothing to request (zeroed again at the use)
                if (STAGE == 1) {
                  ea[kk][cc] = 0u;
                  eb[kk][cc] = 0u;
                } else {
#pragma unroll
                  for (int zs = 0; zs < ZS; ++zs) ez[zs][kk][cc] = v2f{0.f, 0.f};
                }
              } else if (STAGE == 1) {
                ea[kk][cc] = *(const DBF_GLOBAL uint32_t*)((gcp)(f.gamma + ci2 * p.K) + off);
                eb[kk][cc] = *(const DBF_GLOBAL uint32_t*)((gcp)(p.x + t * p.ldx) + off);
              } else {
                // the ZS partial sums of z (one per part of stage 1)
#pragma unroll
                for (int zs = 0; zs < ZS; ++zs)
                  ez[zs][kk][cc] = *(const DBF_GLOBAL v2f*)(
                      (gcp)(zl + zs * p.zpart + ci2 * p.zstride + t * p.ldz) + off);
              }
            }
          }
          if (nk > 0) load_signs();
#pragma unroll
          for (int kk = 0; kk < KC; ++kk)
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) {
              const int64_t k = (kw0 + kk) * kColBlock + 2 * lane;
              const bool on = kk < nk && cc < ncc;
              float v0, v1;
              if (STAGE == 1) {
                const v2h ga = __builtin_bit_cast(v2h, ea[kk][cc]);
                const v2h xb = __builtin_bit_cast(v2h, eb[kk][cc]);
                v0 = (float)ga[0] * (float)xb[0];
                v1 = (float)ga[1] * (float)xb[1];
              } else {
                v0 = ez[0][kk][cc][0];
                v1 = ez[0][kk][cc][1];
#pragma unroll
                for (int zs = 1; zs < ZS; ++zs) {
                  v0 += ez[zs][kk][cc][0];
                  v1 += ez[zs][kk][cc][1];
                }
              }
              ev[kk][cc] = v2f{on && k < p.K ? v0 : 0.0f, on && k + 1 < p.K ? v1 : 0.0f};
            }
        }
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
#pragma unroll
          for (int cc = 0; cc < NCC; ++cc) {
            if (kk >= nk || cc >= ncc) continue;
            const float v0 = ev[kk][cc][0], v1 = ev[kk][cc][1];
            const int col0 = kParts * cc;
            block_parts(v0, v1, [&](int pp, uint16_t code, int sc) {
              *(uint16_t*)(pb + (kk * kPinCols + col0 + pp) * 128 + boff) = code;
              if (lane == 0) ps[kk * kPinCols + col0 + pp] = (uint8_t)(sc + 127);
            });
          }
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          const bool live = colv && kk < nk;
          bop[kk] = live ? *(const v8i*)(pb + (kk * kPinCols + j) * 128 + g * 32)
                         : v8i{0, 0, 0, 0, 0, 0, 0, 0};
          bsc[kk] = live ? (int)ps[kk * kPinCols + j] : 127;
        }
      } else {
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
        if (nk > 0) load_signs();
      }
      if (nk > 0) {
#pragma unroll
        for (int rq = 0; rq < RQ; ++rq) {
          v4f a4[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) a4[h] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KC; ++kk)
#pragma unroll
            for (int h = 0; h < 4; ++h)
              a4[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  expand_signs_fp4(wd[rq][kk][h], p.sign_mask, p.fp4_one), bop[kk], a4[h],
                  4 /* A: fp4 e2m1 */, 0 /* B: fp8 e4m3 */, 0, 127 /* A scale 2^0 */, 0,
                  bsc[kk]);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int rt = 4 * rq + h;
            red[wv][rt][lane] = first_chunk ? a4[h] : red[wv][rt][lane] + a4[h];
          }
        }
      } else if (first_chunk) {
        for (int rt = 0; rt < RTG; ++rt) red[wv][rt][lane] = v4f{0.f, 0.f, 0.f, 0.f};
      }
      first_chunk = false;
    }

    __syncthreads();
    for (int rt = wv; rt < RTG; rt += NW) {
      const int64_t tile = tile0 + rt;
      if (tile >= p.nrt) break;
      v4f sum = red[0][rt][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[w][rt][lane];
      const half_t* srow = (STAGE == 1 ? f.beta : f.alpha) + (int64_t)ci * p.rows;
      half_t scg[4];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        scg[v] = sc_r0 + v < p.rows ? __builtin_bit_cast(half_t, (uint16_t)scu[v]) : (half_t)0.0f;
      gemv_epilogue<STAGE, PIN ? 2 : 0>(p, nsplit > 1 ? zl + ks * p.zpart : zl, yl, srow, sum,
                                        tile, lane, g, part, colv, ci, ct, ntok, t0, scg);
    }
    __syncthreads();
  }
}

template <int STAGE, int RTG, int KC, bool MULTI, bool PIN = false, int NW = 4, bool GROUP = false,
          int ZS = 1>
__global__ __launch_bounds__(64 * NW) void k_gemv_fp4(GemvParams p) {
  __shared__ __attribute__((aligned(16))) char lds[GemvLds<RTG, KC, PIN, NW>::bytes];
  gemv_fp4_items<STAGE, RTG, KC, MULTI, PIN, NW, GROUP, ZS>(p, lds, blockIdx.x, (int)p.grid);
}

// Stage the live B operand pieces of blocks [k0, k0 + nkc) of a column block
// (tokens t0.., ncols = kParts * ell * ntok columns) from the prep output into
// LDS: piece e = ((block * ncols + column) * 4 + g) * 2 + half holds 16 bytes
// at bl + 16 e, and bs[block * 16 + column] the column's scale code.  Blocks
// nkc .. nkc_pad-1 are padding: zero operands with scale 1.0.  Each thread
// issues all loads of a pass before its LDS writes.  Workgroup-wide.
__device__ inline void stage_b(const GemvParams& p, uint8_t* bl, uint8_t* bs, int64_t k0, int nkc,
                               int nkc_pad, int ncols, int ntok, int64_t t0) {
  const int nlive = nkc * ncols * 8;      // < 2^31 (LDS-bounded)
  const int npiece = nkc_pad * ncols * 8;
  const int64_t tb = (int64_t)p.T * p.nkb * (kParts * 4);  // idx stride of one term
  const int64_t ib = ((t0 * p.nkb + k0) * kParts) * 4;     // idx of (term 0, token t0, block k0)
  constexpr int PT = 4;
  for (int e0 = threadIdx.x; e0 < npiece; e0 += PT * (int)blockDim.x) {
    v4u v[PT];
    uint32_t sc[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int e = e0 + q * (int)blockDim.x;
      const int ee = e < nlive ? e : 0;
      const int half = ee & 1, gg = (ee >> 1) & 3;
      const int rest = ee >> 3;
      const int kbl = rest / ncols, col = rest - kbl * ncols;
      const int cc = col / kParts, cpart = col - kParts * cc;
      const int cci = cc / ntok, cct = cc - ntok * cci;
      const int64_t idx =
          cci * tb + ib + ((int64_t)cct * p.nkb + kbl) * (kParts * 4) + cpart * 4 + gg;
      v[q] = *(gv4up)(p.opnd + idx * 8 + half * 4);
      sc[q] = p.oscl[idx];
    }
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int e = e0 + q * (int)blockDim.x;
      if (e < npiece) {
        const bool lv = e < nlive;
        *(v4u*)(bl + e * 16) = lv ? v[q] : v4u{0u, 0u, 0u, 0u};
        if ((e & 7) == 0) {
          const int rest = e >> 3, kbl = rest / ncols;
          bs[kbl * 16 + (rest - kbl * ncols)] = lv ? (uint8_t)sc[q] : (uint8_t)127;
        }
      }
    }
  }
}

// Throughput kernel for many row quads (batched decode over many layers).
// Work item: (column block, group of 4*QPW row quads); wave w of the
// workgroup owns quads w, w+4, ... of the group over the WHOLE reduction, so
// the main loop has no barrier and no cross-wave sum.  Per item, the B
// operands of the live columns are staged once in LDS (in chunks of blocks
// when they do not fit), together with the rows' output scales.  Each lane
// streams its 16-byte A words through a ring of D registers: the load D
// steps ahead is issued as a step is consumed, across quad boundaries (steps
// are padded to a multiple of D per quad; padding and past-the-end loads read
// a clamped in-range address, padding steps meet a zero B operand).  The
// streaming loops hold loads and matrix ops only; tiles are parked in LDS and
// finished by one epilogue loop.
template <int STAGE, int QPW, int D>
__global__ __launch_bounds__(256) void k_gemv_stream(GemvParams p) {
  constexpr int ROWS_ITEM = 4 * QPW * kQuad * kRowTile;  // rows of one item
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // LDS: staged B operands [blocks][live column][g][32 B] (p.lds_b bytes),
  // a 32-byte zero slot for lanes of unused columns, scales [blocks][16]
  // (p.lds_s bytes), per-wave partial tiles [4][QPW][4][64] x 16 B, output
  // scales [ell][ROWS_ITEM].
  uint8_t* bl = smem;
  uint8_t* zslot = smem + p.lds_b;  // 32 zero bytes, then 16 bytes of scale 127
  uint8_t* bs = zslot + 48;
  v4f* partial = (v4f*)(bs + p.lds_s);
  half_t* srows = (half_t*)(partial + 4 * QPW * 4 * 64);
  if (threadIdx.x < 2) *(v4u*)(zslot + 16 * threadIdx.x) = v4u{0u, 0u, 0u, 0u};
  if (threadIdx.x == 2) *(v4u*)(zslot + 32) = v4u{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int c = j / kParts, part = j - kParts * (j / kParts);
  const int64_t n_cb = p.multi ? (int64_t)p.hdr->n_colblocks : p.n_cb_host;
  const int64_t n_items = n_cb * p.n_qg;

  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t cb = it / p.n_qg, qg = it % p.n_qg;
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
    const int64_t qbase = qg * 4 * QPW;
    const int64_t row0 = qbase * kQuad * kRowTile;
    if (ad < 0) {
      if (STAGE == 2 && !p.accumulate) {
        const int64_t nr = (p.rows - row0) < ROWS_ITEM ? (p.rows - row0) : ROWS_ITEM;
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
    const int ntok = (int)(t1 - t0);
    const int ncols = kParts * p.ell * ntok;
    const bool colv = j < ncols;
    const int ci = colv ? c / ntok : 0, ct = colv ? c - ntok * (c / ntok) : 0;
    const char* S = (const char*)(STAGE == 1 ? f.B2 : f.B1);
    const int64_t qw0 = qbase + wv;  // this wave's quads: qw0 + 4*qi
    int nqw = 0;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi)
      if (qw0 + 4 * qi < p.nq) nqw = qi + 1;
    // blocks per chunk: this item's live columns must fit p.lds_b
    // (padded to a multiple of D, which must fit too)
    int64_t kchunk = p.lds_b / ((int64_t)ncols * 128);
    kchunk = kchunk < p.lds_s / 16 ? kchunk : p.lds_s / 16;
    kchunk = kchunk / D * D;
    kchunk = kchunk > D ? kchunk : D;  // D blocks of 16 columns always fit p.lds_b
    kchunk = kchunk < p.nkb ? kchunk : p.nkb;

    for (int64_t k0 = 0; k0 < p.nkb; k0 += kchunk) {
      const int64_t nkc = (p.nkb - k0) < kchunk ? (p.nkb - k0) : kchunk;
      const int64_t nkc_pad = (nkc + D - 1) / D * D;
      __syncthreads();  // every wave is done with the previous chunk's LDS
      // A words: this wave's quads are contiguous runs of 1 KB units; the
      // address is a uniform base plus lane*16 (scalar-base global loads).
      // The first D are requested before the staging below, so their memory
      // latency overlaps the staging's.
      const char* S0 = S + ((qw0 * p.nkb + k0) << 10);
      const int64_t qbytes = (int64_t)4 * p.nkb << 10;  // between this wave's quads
      const int lane16 = lane * 16;
      const int nk = (int)nkc, nkp = (int)nkc_pad;
      v4u ring[D];
      if (nqw > 0) {
#pragma unroll
        for (int u = 0; u < D; ++u) ring[u] = *(gv4up)(S0 + ((u < nk ? u : 0) << 10) + lane16);
      }
      __builtin_amdgcn_sched_barrier(0);
      // output scales of this item's rows for every term (first chunk only),
      // requested together with the B pieces below
      constexpr int kSrPer = (5 * ROWS_ITEM + 255) / 256;  // ell <= 5 on this path
      half_t srv[kSrPer];
      if (k0 == 0) {
        const half_t* sv = STAGE == 1 ? f.beta : f.alpha;
#pragma unroll
        for (int u = 0; u < kSrPer; ++u) {
          const int e = threadIdx.x + u * 256;
          const int i = e / ROWS_ITEM, rr = e - i * ROWS_ITEM;
          srv[u] = (e < p.ell * ROWS_ITEM && row0 + rr < p.rows)
                       ? sv[(int64_t)i * p.rows + row0 + rr] : (half_t)0.0f;
        }
      }
      stage_b(p, bl, bs, k0, (int)nkc, (int)nkc_pad, ncols, ntok, t0);
      if (k0 == 0) {
#pragma unroll
        for (int u = 0; u < kSrPer; ++u) {
          const int e = threadIdx.x + u * 256;
          if (e < p.ell * ROWS_ITEM) srows[e] = srv[u];
        }
      }
      __syncthreads();
      if (nqw == 0) continue;

      v4f acc[QPW][4];
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[qi][h] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        if (qi >= nqw) break;
        const char* cur = S0 + qi * qbytes;
        const bool last_quad = qi + 1 >= nqw;
        const char* nxt = last_quad ? cur : cur + qbytes;
        for (int kb0 = 0; kb0 < nkp; kb0 += D) {
          const bool same = kb0 + D < nkp;
          const char* src = same ? cur : nxt;
          // past the wave's last block the refills re-read that block (just
          // loaded, so a cache hit): their registers are reused after the
          // loop, which waits for them
          const int kn0 = same ? kb0 + D : (last_quad ? nk - 1 : 0);
          // lanes of live columns read [kb][j][g] (padding blocks are staged
          // zeros); the others read the zero slot with stride 0
          const uint8_t* bstep = colv ? bl + ((kb0 * ncols + j) * 4 + g) * 32 : zslot;
          const int bstride = colv ? ncols * 128 : 0;
          const uint8_t* sstep = colv ? bs + kb0 * 16 + j : zslot + 32;
          const int sstride = colv ? 16 : 0;
#pragma unroll
          for (int u = 0; u < D; ++u) {
            // expand the slot's four words, then refill the slot; the refill
            // stays after the last read of the old value so the slot keeps
            // its register (copying an in-flight slot would drain the queue)
            const v4u w = ring[u];
            const v8i a0 = expand_signs_fp4(w[0], p.sign_mask, p.fp4_one);
            const v8i a1 = expand_signs_fp4(w[1], p.sign_mask, p.fp4_one);
            const v8i a2 = expand_signs_fp4(w[2], p.sign_mask, p.fp4_one);
            const v8i a3 = expand_signs_fp4(w[3], p.sign_mask, p.fp4_one);
            __builtin_amdgcn_sched_barrier(0);
            const int kn = (!same && last_quad) ? kn0 : (kn0 + u < nk ? kn0 + u : nk - 1);
            ring[u] = *(gv4up)(src + (kn << 10) + lane16);
            const uint8_t* bp = bstep + u * bstride;
            const v4u lo = *(const v4u*)bp, hi = *(const v4u*)(bp + 16);
            const v8i bop = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int bsc = sstep[u * sstride];
            acc[qi][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, bop, acc[qi][0], 4, 0,
                                                                           0, 127, 0, bsc);
            acc[qi][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, bop, acc[qi][1], 4, 0,
                                                                           0, 127, 0, bsc);
            acc[qi][2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a2, bop, acc[qi][2], 4, 0,
                                                                           0, 127, 0, bsc);
            acc[qi][3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a3, bop, acc[qi][3], 4, 0,
                                                                           0, 127, 0, bsc);
          }
        }
      }
      // park this chunk's tiles in the wave's own LDS partials
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        if (qi >= nqw) break;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v4f* slot = partial + ((wv * QPW + qi) * 4 + h) * 64 + lane;
          *slot = (k0 == 0) ? acc[qi][h] : *slot + acc[qi][h];
        }
      }
    }
    // epilogue of this wave's tiles (its own partials; the scales were
    // staged before the last barrier)
    const half_t* srow = srows + ci * ROWS_ITEM - row0;
#pragma unroll
    for (int e = 0; e < QPW * 4; ++e) {
      const int64_t tile = (qw0 + 4 * (e >> 2)) * kQuad + (e & 3);
      if (e < nqw * 4 && tile < p.nrt)
        gemv_epilogue<STAGE, true>(p, p.z, p.y, srow, partial[(wv * QPW * 4 + e) * 64 + lane], tile, lane, g,
                                   part, colv, ci, ct, ntok, t0);
    }
  }
}

// ------------------------------------------------------- fused decode ----

// Epilogue of one tile in the fused kernel; the arithmetic of gemv_epilogue
// with per-lane row pointers prepared once per column block.  `sum` is this
// lane's MFMA tile (rows r0..r0+3 of column j, r0 = tile*16 + 4g); the parts
// of a column sit in lanes j, j+1, j+2 of one row of 16.  p0: this lane holds
// part 0 of a live column; st: it stores (stage 1: p0; stage 2: p0 and term
// 0).  Stage 1 writes z = beta * u through zrow (fp32, in LDS, rows past the
// last are written too: their scale is zero); stage 2 sums
// alpha_i * w_i over the terms and writes (or accumulates) y through yrow.
// srow: LDS output scales of this lane's term, zero past the rows.  Every
// lane of the wave must call it (it shuffles).
template <int STAGE>
__device__ inline void fused_epilogue(const GemvParams& p, v4f sum, const half_t* srow, int r0,
                                      float* zrow, char* yrow, bool p0, bool st, int g, int lane,
                                      int ntok, int ct) {
  typedef const __attribute__((address_space(3))) v4h* lds_v4hp;
  float tot[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) tot[v] = (sum[v] + row_next<1>(sum[v])) + row_next<2>(sum[v]);
  const v4h s4 = *(lds_v4hp)(srow + r0);
  const int rows = (int)p.rows;
  if (STAGE == 1) {
    typedef __attribute__((address_space(3))) v4f* lds_v4fp;
    if (st)
      *(lds_v4fp)(zrow + r0) = v4f{tot[0] * (float)s4[0], tot[1] * (float)s4[1],
                                   tot[2] * (float)s4[2], tot[3] * (float)s4[3]};
  } else {
    float val[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) val[v] = p0 ? tot[v] * (float)s4[v] : 0.0f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.ell == 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] += val[v];
    } else {
      for (int ii = 0; ii < p.ell; ++ii) {
        int src = 16 * g + kParts * (ii * ntok + ct);
        src = src < 64 ? src : lane;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] += __shfl(val[v], src);
      }
    }
    if (st) {
      if (p.y_f32) {
        float* yr = (float*)yrow + r0;
        if (p.accumulate)
          for (int e = 0; e < 4; ++e) o[e] += r0 + e < rows ? yr[e] : 0.0f;
        if (r0 + 4 <= rows) {
          *(v4f*)yr = v4f{o[0], o[1], o[2], o[3]};
        } else {
          for (int e = 0; e < 4; ++e)
            if (r0 + e < rows) yr[e] = o[e];
        }
      } else {
        half_t* yr = (half_t*)yrow + r0;
        if (p.accumulate)
          for (int e = 0; e < 4; ++e) o[e] += r0 + e < rows ? (float)yr[e] : 0.0f;
        if (r0 + 4 <= rows) {
          *(v4h*)yr = v4h{(half_t)o[0], (half_t)o[1], (half_t)o[2], (half_t)o[3]};
        } else {
          for (int e = 0; e < 4; ++e)
            if (r0 + e < rows) yr[e] = (half_t)o[e];
        }
      }
    }
  }
}

// Streams one stage of a fused column block.  Wave wv starts with row quad
// wv of the stage's sign matrix S and takes each further quad from the
// workgroup's LDS counter *qcnt (which starts at NW) at the start of the
// current one, so the waves a SIMD serves last simply take fewer quads and
// all finish together.  Each quad's four tiles are finished by the epilogue
// right after its last block, while the ring's loads for the next quad are
// in flight.  The ring of D sign loads per lane runs on across quads; after
// the last quad it fetches the first blocks of `tail` (the wave's first quad
// of the next stage, tail_nk blocks long), or re-reads the last block when
// tail is null.
// B operands and their scales come from LDS (bl, bs: blocks padded to a
// multiple of D with zero operands); the epilogue arguments are those of
// fused_epilogue.
template <int STAGE, int D, int NW>
__device__ inline void fused_stream(const GemvParams& p, const char* S, int* qcnt, int wv, int lane,
                                    v4u (&ring)[D], const char* tail, int tail_nk,
                                    const uint8_t* bl, const uint8_t* bs, const uint8_t* zslot,
                                    const half_t* srow, int ncols, bool colv, int j, int g,
                                    float* zrow, char* yrow, bool p0, bool st, int ntok, int ct) {
  const int lane16 = lane * 16;
  const int nk = (int)p.nkb, nkp = (nk + D - 1) / D * D;
  const int nq = (int)p.nq;
  // lanes of live columns read [kb][j][g]; the others read the zero slot
  const uint8_t* bbase = colv ? bl + (j * 4 + g) * 32 : zslot;
  const int bstride = colv ? ncols * 128 : 0;
  const uint8_t* sbase = colv ? bs + j : zslot + 32;
  const int sstride = colv ? 16 : 0;
  for (int q = wv; q < nq;) {
    int qn = 0;
    if (lane == 0) qn = atomicAdd(qcnt, 1);
    qn = __builtin_amdgcn_readfirstlane(qn);
    const char* cur = S + ((int64_t)q * nk << 10);
    const bool lastq = qn >= nq;
    const char* nxt = lastq ? tail : S + ((int64_t)qn * nk << 10);
    const int nxt_nk = lastq ? tail_nk : nk;
    v4f acc[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) acc[h] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < nkp; kb0 += D) {
      const bool same = kb0 + D < nkp;
      const char* src = same ? cur : (nxt != nullptr ? nxt : cur);
      const int kn0 = same ? kb0 + D : (nxt != nullptr ? 0 : nk - 1);
      const int lim = same ? nk : (nxt != nullptr ? nxt_nk : nk);
      const uint8_t* bstep = bbase + kb0 * bstride;
      const uint8_t* sstep = sbase + kb0 * sstride;
#pragma unroll
      for (int u = 0; u < D; ++u) {
        // expand the slot's four words, then refill the slot (the refill
        // stays after the last read of the old value)
        const v4u w = ring[u];
        const v8i a0 = expand_signs_fp4(w[0], p.sign_mask, p.fp4_one);
        const v8i a1 = expand_signs_fp4(w[1], p.sign_mask, p.fp4_one);
        const v8i a2 = expand_signs_fp4(w[2], p.sign_mask, p.fp4_one);
        const v8i a3 = expand_signs_fp4(w[3], p.sign_mask, p.fp4_one);
        __builtin_amdgcn_sched_barrier(0);
        const int kn = kn0 + u < lim ? kn0 + u : lim - 1;
        ring[u] = __builtin_nontemporal_load((gv4up)(src + ((int64_t)kn << 10) + lane16));
        const uint8_t* bp = bstep + u * bstride;
        const v4u lo = *(const v4u*)bp, hi = *(const v4u*)(bp + 16);
        const v8i bop = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const int bsc = sstep[u * sstride];
        acc[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, bop, acc[0], 4, 0, 0, 127, 0, bsc);
        acc[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, bop, acc[1], 4, 0, 0, 127, 0, bsc);
        acc[2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a2, bop, acc[2], 4, 0, 0, 127, 0, bsc);
        acc[3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a3, bop, acc[3], 4, 0, 0, 127, 0, bsc);
      }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int tile = q * kQuad + h;
      if (tile < p.nrt)
        fused_epilogue<STAGE>(p, acc[h], srow, tile * kRowTile + 4 * g, zrow, yrow, p0, st, g,
                              lane, ntok, ct);
    }
    q = qn;
  }
}

// Inputs of the fused kernel besides the two stages' parameters.
struct FusedArgs {
  int32_t rows_pad;  // output-scale rows staged per term: max(R, N) rounded up to 64
  int32_t rz;        // z entries kept per (term, token): R rounded up to 128
  int32_t n_slots;   // column blocks one workgroup can own: ceil(max blocks / grid)
  int32_t chunk;     // tokens per column block at most
  int32_t num_adapters;
  const int32_t* ids;
  const half_t* x;
  int64_t ldx;
  const half_t* const* gammas;
};

// Writes the fp8 parts of the operand columns (term i, token tt) of block kb
// into the LDS operand area, from the two entries v0, v1 (block cols 2*lane,
// 2*lane+1) of this lane; the arithmetic of the prep kernel.  Wave-wide.
__device__ inline void parts_to_lds(float v0, float v1, uint8_t* bl, uint8_t* bs, int kb, int col0,
                                    int ncols, int lane) {
  uint8_t* dst = bl + ((int64_t)kb * ncols + col0) * 128 + fp8_operand_byte(operand_k_of_col(2 * lane));
  block_parts(v0, v1, [&](int pp, uint16_t code, int sc) {
    *(uint16_t*)(dst + pp * 128) = code;
    if (lane == 0) bs[kb * 16 + col0 + pp] = (uint8_t)(sc + 127);
  });
}

// Zero operands with scale 1.0 for the padding blocks [nk, nkp).  Workgroup-wide.
__device__ inline void pad_blocks(uint8_t* bl, uint8_t* bs, int nk, int nkp, int ncols) {
  for (int e = threadIdx.x; e < (nkp - nk) * ncols * 8; e += blockDim.x)
    *(v4u*)(bl + ((int64_t)nk * ncols * 8 + e) * 16) = v4u{0u, 0u, 0u, 0u};
  for (int e = threadIdx.x; e < (nkp - nk) * 16; e += blockDim.x) bs[nk * 16 + e] = 127;
}

// The whole multi-adapter product for many column blocks (batched decode)
// in one launch.  Each workgroup segments the ids itself (every workgroup
// finds the same list) and keeps the column blocks b, b + G, ... (G =
// workgroups); for each it builds the stage-1 operands gamma_i * x in fp8
// parts directly in LDS, streams stage 1 over every row quad of its adapter
// (z = beta * u stays in LDS, fp32; the workspace is not used), turns its
// z into the stage-2 parts in LDS, and streams stage 2.  No other launch, no other
// workgroup and no per-item set-up lies between the steps, and the stage-1
// ring ends by fetching the first stage-2 sign blocks.  The parts are those
// of the prep kernel, so the result equals the split-phase path's.  p1/p2
// describe stage 1 (rows R, reduction M) and stage 2 (rows N, reduction R).
// NW waves per workgroup: with one column block per compute unit, several
// waves per SIMD hide each other's LDS and matrix-core latencies.  The sign
// words are read once, so their loads are non-temporal.
// LDS: B operands [blocks][column][g][32 B] (p1.lds_b bytes), a 48-byte slot
// (32 zero bytes, 16 bytes of scale code 127), operand scales [blocks][16]
// (p1.lds_s bytes), output scales of stage 1 and of stage 2 [ell][rows_pad]
// halfs each, column blocks [n_slots], z [ell * chunk][rz] fp32.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemv_fused(GemvParams p1, GemvParams p2,
                                                        FusedArgs fx) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* bl = smem;
  uint8_t* zslot = smem + p1.lds_b;
  uint8_t* bs = zslot + 48;
  half_t* srows = (half_t*)(bs + p1.lds_s);                // beta
  half_t* srows2 = srows + (int64_t)p1.ell * fx.rows_pad;  // alpha
  ColBlock* cbs = (ColBlock*)(srows2 + (int64_t)p1.ell * fx.rows_pad);
  float* zl = (float*)(cbs + fx.n_slots);
  __shared__ int qcnt[2];  // next row quad to take, per stage
  if (threadIdx.x < 2) *(v4u*)(zslot + 16 * threadIdx.x) = v4u{0u, 0u, 0u, 0u};
  if (threadIdx.x == 2) *(v4u*)(zslot + 32) = v4u{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int c = j / kParts, part = j - kParts * (j / kParts);
  const int lane16 = lane * 16;
  const int ell = p1.ell;
  const int nkb1 = (int)p1.nkb, nkb2 = (int)p2.nkb;
  const int nkp1 = (nkb1 + D - 1) / D * D, nkp2 = (nkb2 + D - 1) / D * D;
  const bool has1 = wv < p1.nq, has2 = wv < p2.nq;  // a first quad in each stage
  const int G = gridDim.x, b = blockIdx.x;

  const int32_t n_cb = segment_runs<NW>(
      fx.ids, (int32_t)p1.T, fx.num_adapters, fx.chunk,
      [&](int32_t idx, int32_t t, int32_t id) {
        if (idx % G == b) {
          cbs[idx / G].t0 = t;
          cbs[idx / G].adapter = id;
        }
      },
      [&](int32_t idx, int32_t t1) {
        if (idx % G == b) cbs[idx / G].t1 = t1;
      });
  __syncthreads();  // the slots were written by the block-start threads

  int slot = 0;
  for (int32_t cb = b; cb < n_cb; cb += G, ++slot) {
    const ColBlock cbk = cbs[slot];
    const int64_t t0 = cbk.t0, t1 = cbk.t1;
    const int32_t ad = cbk.adapter;
    if (ad < 0) {  // out-of-range ids: y = 0 (or unchanged)
      if (!p2.accumulate) {
        const int64_t nr = p2.rows;
        for (int64_t e = threadIdx.x; e < (t1 - t0) * nr; e += blockDim.x) {
          const int64_t t = t0 + e / nr, r = e % nr;
          if (p2.y_f32)
            ((float*)p2.y)[t * p2.ldy + r] = 0.0f;
          else
            ((half_t*)p2.y)[t * p2.ldy + r] = (half_t)0.0f;
        }
      }
      continue;
    }
    const uint32_t* B1 = p1.B1s[ad];
    const uint32_t* B2 = p1.B2s[ad];
    const half_t* alpha = p1.alphas[ad];
    const half_t* beta = p1.betas[ad];
    const half_t* gamma = fx.gammas[ad];
    const int ntok = (int)(t1 - t0);
    const int ncols = kParts * ell * ntok;
    const bool colv = j < ncols;
    const int ci = colv ? c / ntok : 0, ct = colv ? c - ntok * (c / ntok) : 0;
    const char* S1 = (const char*)B2;
    const char* S2 = (const char*)B1;
    const char* S1w = S1 + ((int64_t)wv * nkb1 << 10);  // this wave's first quads
    const char* S2w = S2 + ((int64_t)wv * nkb2 << 10);
    const bool p0 = part == 0 && colv;
    float* zrow = zl + (ci * ntok + ct) * fx.rz;
    char* yrow = (char*)p2.y + (t0 + ct) * p2.ldy * (p2.y_f32 ? 4 : 2);

    // ---- stage 1 operands v_i = gamma_i * x (exact in fp32) in fp8 parts:
    // wave tasks (term, token, block), four tasks' loads requested together.
    // The first four tasks are requested before the first D sign loads, so
    // their parts need not wait for the signs.
    const int ntask1 = ell * ntok * nkb1;
    const int M = (int)p1.K;
    // Each entry is a 16-bit load from an address clamped into its row, kept
    // zero-extended in a register of its own until parts_v: no branch,
    // packing or arithmetic next to the requests, so the sign ring below is
    // requested while they are in flight.
    typedef const DBF_GLOBAL uint16_t* gu16p;
    auto load_v = [&](int task0, uint32_t (&e)[4][4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int task = task0 + q * NW, tq = task < ntask1 ? task : ntask1 - 1;
        const int kb = tq % nkb1, cc = tq / nkb1;  // cc = term * ntok + token
        const int i = cc / ntok, tt = cc - i * ntok;
        const int k = kb * kColBlock + 2 * lane;
        const int k0 = k < M ? k : M - 1, k1 = k + 1 < M ? k + 1 : M - 1;
        const half_t* xr = fx.x + (t0 + tt) * fx.ldx;
        const half_t* gi = gamma + (int64_t)i * M;
        e[q][0] = *(gu16p)(gi + k0);
        e[q][1] = *(gu16p)(gi + k1);
        e[q][2] = *(gu16p)(xr + k0);
        e[q][3] = *(gu16p)(xr + k1);
      }
    };
    auto parts_v = [&](int task0, const uint32_t (&e)[4][4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int task = task0 + q * NW;
        if (task < ntask1) {
          const int k = (task % nkb1) * kColBlock + 2 * lane;
          auto h = [&](int w) { return (float)__builtin_bit_cast(half_t, (uint16_t)e[q][w]); };
          const float v0 = k < M ? h(0) * h(2) : 0.0f, v1 = k + 1 < M ? h(1) * h(3) : 0.0f;
          parts_to_lds(v0, v1, bl, bs, task % nkb1, (task / nkb1) * kParts, ncols, lane);
        }
      }
    };
    uint32_t ev[4][4];
    load_v(wv, ev);
    v4u ring[D];
    if (has1) {
#pragma unroll
      for (int u = 0; u < D; ++u)
        ring[u] = *(gv4up)(S1w + ((int64_t)(u < nkb1 ? u : nkb1 - 1) << 10) + lane16);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // the previous column block's LDS readers are done
    if (threadIdx.x == 0) qcnt[0] = qcnt[1] = NW;
    parts_v(wv, ev);
    for (int task0 = wv + 4 * NW; task0 < ntask1; task0 += 4 * NW) {
      load_v(task0, ev);
      parts_v(task0, ev);
    }
    pad_blocks(bl, bs, nkb1, nkp1, ncols);
    // output scales of both stages, kSc per thread requested together (a
    // load-then-store loop would pay one loaded round trip per element)
    {
      constexpr int kSc = 8;
      const int nsc = ell * fx.rows_pad;
      for (int e0 = threadIdx.x; e0 < nsc; e0 += kSc * (int)blockDim.x) {
        half_t vb[kSc], va[kSc];
#pragma unroll
        for (int u = 0; u < kSc; ++u) {
          const int e = e0 + u * (int)blockDim.x;
          const int i = e / fx.rows_pad, r = e - i * fx.rows_pad;
          vb[u] = (e < nsc && r < p1.rows) ? beta[(int64_t)i * p1.rows + r] : (half_t)0.0f;
          va[u] = (e < nsc && r < p2.rows) ? alpha[(int64_t)i * p2.rows + r] : (half_t)0.0f;
        }
#pragma unroll
        for (int u = 0; u < kSc; ++u) {
          const int e = e0 + u * (int)blockDim.x;
          if (e < nsc) {
            srows[e] = vb[u];
            srows2[e] = va[u];
          }
        }
      }
    }
    __syncthreads();
    fused_stream<1, D, NW>(p1, S1, &qcnt[0], wv, lane, ring, has2 ? S2w : nullptr, nkb2, bl, bs,
                           zslot, srows + ci * fx.rows_pad, ncols, colv, j, g, zrow, yrow, p0, p0,
                           ntok, ct);

    // ---- z of this column block is complete once every wave is past this
    // barrier
    __syncthreads();
    if (!has1 && has2) {
#pragma unroll
      for (int u = 0; u < D; ++u)
        ring[u] = *(gv4up)(S2w + ((int64_t)(u < nkb2 ? u : nkb2 - 1) << 10) + lane16);
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      // stage-2 operands from z, wave tasks (term, token, block)
      const int ntask = ell * ntok * nkb2;
      const int R = (int)p1.rows;
      for (int task0 = wv; task0 < ntask; task0 += 4 * NW) {
        float v0[4], v1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int task = task0 + q * NW;
          v0[q] = v1[q] = 0.0f;
          if (task < ntask) {
            const int kb = task % nkb2, cc = task / nkb2;
            const int i = cc / ntok, tt = cc - i * ntok;
            const float* zr = zl + (i * ntok + tt) * fx.rz;
            const int k = kb * kColBlock + 2 * lane;
            if (k < R) v0[q] = zr[k];
            if (k + 1 < R) v1[q] = zr[k + 1];
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int task = task0 + q * NW;
          if (task < ntask)
            parts_to_lds(v0[q], v1[q], bl, bs, task % nkb2, (task / nkb2) * kParts, ncols, lane);
        }
      }
      pad_blocks(bl, bs, nkb2, nkp2, ncols);
    }
    __syncthreads();
    fused_stream<2, D, NW>(p2, S2, &qcnt[1], wv, lane, ring, nullptr, 0, bl, bs, zslot,
                           srows2 + ci * fx.rows_pad, ncols, colv, j, g, zrow, yrow, p0,
                           p0 && ci == 0, ntok, ct);
  }
}

// -------------------------------------------------------------- launch ----

template <int STAGE, int RTG, int KC>
static hipError_t launch_gemv_stage(GemvParams p, int64_t grid, hipStream_t s) {
  if ((p.multi ? max_colblocks(p.T) : p.n_cb_host) * p.n_rg > INT32_MAX) return hipErrorInvalidValue;
  p.grid = grid;
  if (p.multi)
    hipLaunchKernelGGL((k_gemv_fp4<STAGE, RTG, KC, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemv_fp4<STAGE, RTG, KC, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Tile choice: KC reduction blocks per wave chunk (8, or 4 when the four
// waves would otherwise idle), RTG row tiles per item with RTG*KC <= 64 sign
// words per lane in flight; fewer row tiles per item when there are too few
// items to fill the GPU.
constexpr int kFusedD = 8;                    // fused kernel: sign loads in flight per lane
constexpr int kFusedNW = 12;                  // fused kernel: waves per workgroup
constexpr int64_t kFusedMinColBlocks = 256;   // one per compute unit
constexpr int64_t kFusedLdsMax = 160 * 1024;  // LDS budget: one workgroup per compute unit
constexpr int kStreamQPW = 2;  // row quads per wave and item
constexpr int kStreamD = 8;    // sign loads in flight per lane
constexpr int64_t kStreamLdsB = 32 * 1024;  // LDS budget for staged B operands
constexpr int64_t kPinSplitWorkgroups = 256;  // split decode stage 1: one per compute unit

// A stage that builds its own operand parts: 16 waves per workgroup, so a
// wave's chunk is kc = 1, 2 or 4 blocks (4: one adapter, not grouped), one
// quad of row tiles per item (stage 1: per part of its reduction).  An item
// of at most 4 blocks runs 4 waves instead (one block each): 16 would leave
// most waves idle, and the workgroup's barrier would still wait for the
// last of them to be launched.
template <int STAGE, int KC, bool GROUP, int ZS, int NW = 16>
static void launch_pin_k(const GemvParams& p, hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_fp4<STAGE, 4, KC, false, true, NW, GROUP, ZS>), dim3((unsigned)p.grid),
                     dim3(64 * NW), 0, s, p);
}

template <int KC, bool GROUP, int NW>
static hipError_t launch_pin_stage2(const GemvParams& p, int zs, hipStream_t s) {
  // ZS * KC <= 8: at most 16 pairs of z entries per lane in flight
  if (zs == 1) launch_pin_k<2, KC, GROUP, 1, NW>(p, s);
  else if (zs == 2) launch_pin_k<2, KC, GROUP, 2, NW>(p, s);
  else if constexpr (KC <= 2) {
    if (zs == 4) launch_pin_k<2, KC, GROUP, 4, NW>(p, s);
    else if constexpr (KC == 1) {
      if (zs == 8) launch_pin_k<2, KC, GROUP, 8, NW>(p, s);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// zs: stage 1, the parts of its reduction (p.ksplit); stage 2, the partial
// sums of z to add.
template <int STAGE>
static hipError_t launch_gemv_pin(GemvParams p, int kc, int zs, hipStream_t s) {
  p.nq = cdiv(p.nrt, kQuad);
  p.n_rg = cdiv(p.nrt, kQuad);
  const int64_t grid =
      p.n_cb_host * p.n_rg * (p.group > 1 ? p.group : 1) * (STAGE == 1 ? zs : 1);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  p.grid = grid;
  // blocks of one item
  const int64_t nbk = STAGE == 1 && zs > 1 ? p.kslice : p.nkb;
  const bool nw4 = nbk <= 4;
  if (STAGE == 2) {
    if (p.group > 1) {
      if (nw4) return launch_pin_stage2<1, true, 4>(p, zs, s);
      return kc == 1 ? launch_pin_stage2<1, true, 16>(p, zs, s)
                     : launch_pin_stage2<2, true, 16>(p, zs, s);
    }
    if (nw4) return launch_pin_stage2<1, false, 4>(p, zs, s);
    return kc == 1 ? launch_pin_stage2<1, false, 16>(p, zs, s)
           : kc == 4 ? launch_pin_stage2<4, false, 16>(p, zs, s)
                     : launch_pin_stage2<2, false, 16>(p, zs, s);
  }
  if (p.group > 1) {
    if (nw4) launch_pin_k<1, 1, true, 1, 4>(p, s);
    else if (kc == 1) launch_pin_k<1, 1, true, 1>(p, s);
    else launch_pin_k<1, 2, true, 1>(p, s);
  } else if (nw4) {
    launch_pin_k<1, 1, false, 1, 4>(p, s);
  } else if (kc == 1) {
    launch_pin_k<1, 1, false, 1>(p, s);
  } else if (kc == 4) {
    launch_pin_k<1, 4, false, 1>(p, s);
  } else {
    launch_pin_k<1, 2, false, 1>(p, s);
  }
  return hipGetLastError();
}

template <int STAGE>
static hipError_t launch_gemv_stage_any(GemvParams p, int64_t n_cb_est, int64_t n_cb_max,
                                        bool multi, hipStream_t s) {
  p.nq = cdiv(p.nrt, kQuad);
  if (n_cb_est * p.nq >= 1024) {
    // many quads: streaming kernel
    p.lds_b = kStreamLdsB;
    p.lds_s = 16 * (cdiv(p.nkb, 8) * 8 < 256 ? cdiv(p.nkb, 8) * 8 : 256);
    p.n_qg = cdiv(p.nq, 4 * kStreamQPW);
    const size_t lds = (size_t)p.lds_b + 48 + (size_t)p.lds_s +
                       (size_t)4 * kStreamQPW * 4 * 64 * 16 +
                       (size_t)p.ell * 4 * kStreamQPW * kQuad * kRowTile * sizeof(half_t);
    int64_t grid = n_cb_max * p.n_qg;
    if (grid > 2048) grid = 2048;
    hipLaunchKernelGGL((k_gemv_stream<STAGE, kStreamQPW, kStreamD>), dim3((unsigned)grid), dim3(256), lds, s,
                       p);
    return hipGetLastError();
  }
  if (!multi && p.nkb > 4 * 8) {
    // few column blocks and a reduction longer than one round of 4 waves x
    // 8 blocks: 16 waves split it, 4 blocks each per round, so an item
    // makes half as many dependent rounds (one quad of row tiles per item)
    p.n_rg = cdiv(p.nrt, kQuad);
    const int64_t grid = n_cb_max * p.n_rg;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    p.grid = grid;
    hipLaunchKernelGGL((k_gemv_fp4<STAGE, 4, 4, false, false, 16>), dim3((unsigned)grid), dim3(1024),
                       0, s, p);
    return hipGetLastError();
  }
  const int kc = p.nkb > 16 ? 8 : 4;
  const int rtg_max = 64 / kc;
  int rtg = 4;
  if (n_cb_est * cdiv(p.nrt, rtg_max) >= 1024) rtg = rtg_max;
  p.n_rg = cdiv(p.nrt, rtg);
  int64_t grid = n_cb_max * p.n_rg;
  if (multi && grid > 4096) grid = 4096;
  if (kc == 8) {
    if (rtg == 8) return launch_gemv_stage<STAGE, 8, 8>(p, grid, s);
    return launch_gemv_stage<STAGE, 4, 8>(p, grid, s);
  }
  if (rtg == 16) return launch_gemv_stage<STAGE, 16, 4>(p, grid, s);
  return launch_gemv_stage<STAGE, 4, 4>(p, grid, s);
}

static hipError_t launch_prep(PrepParams p, hipStream_t s) {
  const int64_t nblk = (int64_t)p.ell * p.T * p.nkb;
  if (nblk > INT32_MAX - 8) return hipErrorInvalidValue;
  const int64_t grid = cdiv(nblk, 4) + (p.seg_cbl != nullptr ? 1 : 0);
  if (p.multi)
    hipLaunchKernelGGL(k_prep<true>, dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_prep<false>, dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv(const ForwardArgs& a, hipStream_t s) {
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  const int tcb = gemv_tokens_per_block(a.ell);
  hipError_t e;
  int64_t n_cb_max, n_cb_est;
  if (a.multi) {
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
  gp.sign_mask = 0x88888888u;
  gp.fp4_one = 0x22222222u;
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

  GemvParams g1 = gp;
  g1.rows = a.R;
  g1.K = a.M;
  g1.nrt = cdiv(a.R, kRowTile);
  g1.nkb = cdiv(a.M, kColBlock);
  GemvParams g2 = gp;
  g2.rows = a.N;
  g2.K = a.R;
  g2.nrt = cdiv(a.N, kRowTile);
  g2.nkb = cdiv(a.R, kColBlock);

  // many column blocks and every phase in this call: one fused launch when
  // a column block's operands and output scales fit in LDS
  if (a.multi && a.phases == 7 && n_cb_est >= kFusedMinColBlocks) {
    const int64_t nkp = cdiv(g1.nkb > g2.nkb ? g1.nkb : g2.nkb, kFusedD) * kFusedD;
    const int64_t rows_pad = cdiv(a.R > a.N ? a.R : a.N, 64) * 64;
    // one workgroup per compute unit: extra workgroups (the host only
    // bounds the count) would wait for a free unit and end the launch late
    const int64_t grid = n_cb_max < kFusedMinColBlocks ? n_cb_max : kFusedMinColBlocks;
    const int64_t n_slots = cdiv(max_colblocks(a.T), grid);
    const int64_t lds_b = (int64_t)kParts * a.ell * tcb * nkp * 128;
    const int64_t lds_s = 16 * nkp;
    const int64_t rz = cdiv(a.R, kColBlock) * kColBlock;
    const int64_t lds = lds_b + 48 + lds_s + 2 * (int64_t)a.ell * rows_pad * (int64_t)sizeof(half_t) +
                        n_slots * (int64_t)sizeof(ColBlock) + (int64_t)a.ell * tcb * rz * 4;
    // the kernel's static LDS (its id counters and segmentation arrays)
    // shares the budget with the dynamic part
    hipFuncAttributes fa{};
    const bool fa_ok =
        hipFuncGetAttributes(&fa, (const void*)k_gemv_fused<kFusedD, kFusedNW>) == hipSuccess;
    const int64_t lds_static = fa_ok ? (int64_t)fa.sharedSizeBytes : 4096;
    if (lds + lds_static <= kFusedLdsMax) {
      g1.nq = cdiv(g1.nrt, kQuad);
      g2.nq = cdiv(g2.nrt, kQuad);
      g1.lds_b = g2.lds_b = lds_b;
      g1.lds_s = g2.lds_s = lds_s;
      FusedArgs fx{};
      fx.rows_pad = (int32_t)rows_pad;
      fx.rz = (int32_t)rz;
      fx.n_slots = (int32_t)n_slots;
      fx.chunk = tcb;
      fx.num_adapters = a.num_adapters;
      fx.ids = a.ids;
      fx.x = a.x;
      fx.ldx = a.ldx;
      fx.gammas = a.gammas;
      hipLaunchKernelGGL((k_gemv_fused<kFusedD, kFusedNW>), dim3((unsigned)grid),
                         dim3(64 * kFusedNW), (size_t)lds, s, g1, g2, fx);
      return hipGetLastError();
    }
  }

  // With one adapter and at most two columns per operand part (ell *
  // tokens <= 2, the decode case), a stage whose reduction is at most 64
  // blocks (32 when grouped) builds its operand parts itself (0: a prep
  // launch does).  Every workgroup builds the parts of the whole reduction,
  // so this pays only while that is short: at 50 blocks (4 per wave) it
  // saves the prep launch by a small margin.
  auto pin_kc = [&](int64_t nkb) -> int {
    const int64_t ntok = a.T < tcb ? a.T : tcb;
    if (a.multi || (int64_t)a.ell * ntok > kPinColTokens) return 0;
    return nkb <= 16 ? 1 : nkb <= 32 ? 2 : (nkb <= 64 && a.group <= 1) ? 4 : 0;
  };
  // stage 1 reads gamma and x as aligned pairs of entries: M even and every
  // gamma 4-byte aligned (x rows are 16-byte aligned by the boundary's rules)
  bool pairs1 = a.M % 2 == 0;
  for (int j = 0; j < (a.group > 1 ? a.group : 1); ++j)
    pairs1 = pairs1 && (((uintptr_t)(a.group > 1 ? a.grp[j].gamma : a.single.gamma)) & 3u) == 0;
  const int kc2 = pin_kc(g2.nkb);
  // With stage 2 building its parts from z, stage 1 splits its reduction
  // into zs parts (a power of two, each non-empty, at most kMaxZParts / kc2
  // so that stage 2's requests of the partial sums stay in registers): as
  // many as keep one workgroup per compute unit, and at least enough for a
  // part to build its own parts (32 blocks; 64 with one operand column when
  // stage 2 takes 4 blocks per wave, which grouped calls never do; with two
  // columns a 64-block part measured slower than the prep launch).  The
  // choice does not depend on the number of grouped layers, so a grouped
  // call's z is bit for bit that of the single calls.
  int zs = 1;
  if (pairs1 && kc2 > 0) {
    const int smax = kMaxZParts / kc2;
    const int64_t pin_cols = (int64_t)a.ell * (a.T < tcb ? a.T : tcb);
    const int64_t lim = kc2 == 4 && pin_cols == 1 ? 64 : 32;
    const int64_t items = n_cb_max * cdiv(g1.nrt, kQuad);
    int sp = 1;
    while (sp < smax && cdiv(g1.nkb, sp) > lim) sp *= 2;
    if (cdiv(g1.nkb, sp) <= lim) {
      while (2 * sp <= smax && 2 * sp <= g1.nkb && items * 2 * sp <= kPinSplitWorkgroups) sp *= 2;
      while (sp > 1 && (sp - 1) * cdiv(g1.nkb, sp) >= g1.nkb) sp /= 2;
      zs = sp;
    }
  }
  const int64_t kslice = cdiv(g1.nkb, zs);
  const int kc1 = pairs1 ? pin_kc(kslice) : 0;
  g1.ksplit = zs;
  g1.kslice = (int32_t)kslice;
  g1.zpart = g2.zpart = (int64_t)a.ell * a.T * ldz;
  if (a.group > 1) {
    // one launch per stage for every layer when both stages build their own
    // parts; otherwise the caller runs the layers one by one (nothing has
    // been launched)
    if (kc1 == 0 || kc2 == 0) return hipErrorNotSupported;
    for (GemvParams* q : {&g1, &g2}) {
      q->group = a.group;
      q->layer_ws = (int64_t)a.layer_ws;
      q->y_layer_bytes = a.y_layer_bytes;
      for (int j = 0; j < a.group; ++j) q->grp[j] = a.grp[j];
    }
  }

  // stage 1: z = beta * (S2 . (gamma * x))
  if (kc1 > 0) {
    g1.x = a.x;
    g1.ldx = a.ldx;
    if ((a.phases & 2) && (e = launch_gemv_pin<1>(g1, kc1, zs, s)) != hipSuccess) return e;
  } else {
    pp.K = a.M;
    pp.nkb = cdiv(a.M, kColBlock);
    pp.from_z = 0;
    pp.opnd = (uint32_t*)(ws + L.p1o);
    pp.oscl = (uint8_t*)(ws + L.p1s);
    if (a.multi) {  // the first prep launch also builds the column blocks
      pp.seg_cbl = (ColBlock*)(ws + L.cbl);
      pp.seg_hdr = (WsHeader*)ws;
      pp.seg_chunk = tcb;
    }
    if ((a.phases & 1) && (e = launch_prep(pp, s)) != hipSuccess) return e;
    pp.seg_cbl = nullptr;
    g1.opnd = pp.opnd;
    g1.oscl = pp.oscl;
    if ((a.phases & 2) &&
        (e = launch_gemv_stage_any<1>(g1, n_cb_est, n_cb_max, a.multi, s)) != hipSuccess)
      return e;
  }
  if (!(a.phases & 4)) return hipSuccess;
  if (kc2 > 0) return launch_gemv_pin<2>(g2, kc2, zs, s);

  // stage 2: y = sum_i alpha_i * (S1 . z_i)
  pp.K = a.R;
  pp.nkb = cdiv(a.R, kColBlock);
  pp.from_z = 1;
  pp.opnd = (uint32_t*)(ws + L.p2o);
  pp.oscl = (uint8_t*)(ws + L.p2s);
  if ((e = launch_prep(pp, s)) != hipSuccess) return e;
  g2.opnd = pp.opnd;
  g2.oscl = pp.oscl;
  return launch_gemv_stage_any<2>(g2, n_cb_est, n_cb_max, a.multi, s);
}

}  // namespace dbf
