// Large-T (prefill) path: the two sign-accumulation stages as fp16 matrix-
// core contractions.
//
// Once the signs are expanded to +-1 each stage is a dense contraction over
// the batch (DBF summary, section 2, inference: the product with the weight
// becomes two products with sign matrices), so it runs on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation; the operands v_i =
// gamma_i*x and z_i = beta_i*u_i are rounded to fp16 once each.
//
// Launches: prep (v_i = gamma_i * x; with several adapters one extra
// workgroup also builds the column blocks) -> stage 1 (z_i = beta_i * B2 v_i)
// -> stage 2 (y = sum_i alpha_i * B1 z_i).  With one adapter, M a multiple
// of 8 and gamma 16-byte aligned there is no prep launch: stage 1 reads x in
// place as its token operand and folds gamma_i into the expanded signs,
// +-gamma_i[m] being exact in fp16, so the products gamma*x*(+-1) are exact
// in the fp32 accumulation (the prep path rounds gamma*x to fp16 once).
// v and z live in the workspace in
// MFMA operand order: tiles of 16 tokens x 128 reduction entries, 4 KB each
// (4 steps x 64 lanes x 8), so every operand load of a wave is 1 KB
// contiguous, and entries past the reduction length are zero, so the last
// block needs no masking (the padding signs are +1).
//
// K order: the packed word a lane of group g holds for (row rho, 128-block)
// supplies the A operand of four 32-K steps s = 0..3, slots 8s..8s+7 each
// (bits s, s+4, ..., s+28), which are the block cols 32s + 8g + e, e = 0..7.
// The operand tiles put entry 32s + 8g + e of token c16 in lane 16g + c16 of
// step s, so both operands see the same k and no lane exchange is needed.
//
// Stage 3 (the backward pass's sign products) is stage 2 without output
// scales: each term's raw fp32 product S * opnd_i is written to its own
// [T][ldy] block of y.
//
// Work item: a column block of 16*NC tokens and either one row quad (64
// rows) whose reduction the NWV waves split (SPLITK: interleaved 128-blocks,
// partial tiles summed in a fixed order through LDS; 8 waves when there are
// no more items than compute units, so two waves share each SIMD), or four
// row quads, one per wave, each over the whole reduction (for short
// reductions).  Output
// column j of an MFMA depends only on operand column j, so columns of tokens
// past the block's end read a valid token's tile row and are simply not
// stored.
#include <climits>

#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

namespace {

typedef const DBF_GLOBAL v8h* gv8hp;

struct GemmParams {
  int32_t rows, K, T, nq, nkb, ell;
  int32_t n_cb_host, n_rg;  // column blocks (single adapter; an estimate with several), row groups
  int32_t y_f32, accumulate, multi, xcd_remap;
  int32_t grid;             // workgroups launched
  uint32_t msk16, one16;  // 0x80008000, 0x3C003C00 (kept in registers)
  const half_t* x;        // stage 1 reading x in place: token rows, stride ldx
  int64_t ldx;
  const half_t* opnd;     // this stage's operand tiles (v or z)
  int64_t opnd_term;      // halfs per term
  int32_t opnd_nkb;       // 128-blocks per token tile row of the operand
  int32_t z_nkb;          // stage 1: 128-row blocks of z
  half_t* z;              // stage 1 output tiles
  int64_t z_term;
  void* y;
  int64_t ldy;
  int64_t y_term;  // stage 3: floats per term of the output
  Factors single;
  // grouped same-input layers: work items of layer j follow those of j-1;
  // layer j reads grp[j], and offsets z / opnd by j*layer_ws bytes, y by
  // j*y_layer_bytes
  int32_t group;
  int64_t layer_ws, y_layer_bytes;
  Factors grp[kMaxGroup];
  const ColBlock* cbl;
  const WsHeader* hdr;
  int32_t cb_cap;        // column-block entries the workspace holds
  int32_t num_adapters;  // several adapters: entries of the pointer tables
  const uint32_t* const* B1s;
  const uint32_t* const* B2s;
  const half_t* const* alphas;
  const half_t* const* betas;
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

// As expand_step_f16 with the magnitudes of a scale vector along K: the
// sign bits are XORed into gam (the lane's 8 entries of gamma_i for this
// step, two per word), giving +-gamma exactly.
template <int s>
__device__ inline v8h expand_step_gamma(uint32_t w, uint32_t msk, const v4u& gam) {
  const uint32_t U = w << (7 - s), V = w << (3 - s);
  v4u o;
  o[0] = (__builtin_amdgcn_perm(V, U, 0x040C000Cu) & msk) ^ gam[0];
  o[1] = (__builtin_amdgcn_perm(V, U, 0x050C010Cu) & msk) ^ gam[1];
  o[2] = (__builtin_amdgcn_perm(V, U, 0x060C020Cu) & msk) ^ gam[2];
  o[3] = (__builtin_amdgcn_perm(V, U, 0x070C030Cu) & msk) ^ gam[3];
  return __builtin_bit_cast(v8h, o);
}

// Operands of one 128-block: sign words of the four row tiles, the operand
// b[s][c] of step s for token column c and, when stage 1 reads x in place,
// gamma_i at the lane's 8 entries of each step.
template <int NC, bool XIN>
struct Block {
  v4u a;
  v8h b[4][NC];
  v4u gm[XIN ? 4 : 1];
};

// orow[c]: the lane's 16 bytes of token column c's tile row; step s of
// block kb sits at orow[c] + kb*2048 + s*512.
template <int NC>
__device__ inline void load_block(Block<NC, false>& B, const char* sq,
                                  const half_t* const (&orow)[NC], int kb) {
  B.a = *(gv4up)(sq + ((int64_t)kb << 10));
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int c = 0; c < NC; ++c) B.b[s][c] = *(gv8hp)(orow[c] + (int64_t)kb * 2048 + s * 512);
}

// x read in place.  The MFMA operand puts 16 tokens in 16 adjacent lanes, so
// loading it straight from the rows of x would touch 16 half-used cache
// lines per 16 lanes.  Instead lane L loads 16-byte chunk L%16 of rows L/16,
// L/16 + 4, ... of the block's 16*NC tokens (b, read as a flat array: 256
// contiguous bytes per 16 lanes), and x_to_operand passes them through the
// wave's own LDS area into operand order.  grow is entry 8g of gamma_i, so
// step s of block kb needs the 8 gamma entries at kb*128 + 32s (16 bytes,
// aligned as M is a multiple of 8).  A whole block (128 kb + 128 <= M):
template <int NC>
__device__ inline void load_block(Block<NC, true>& B, const char* sq,
                                  const half_t* const (&xrow)[4 * NC], const half_t* grow,
                                  int kb) {
  B.a = *(gv4up)(sq + ((int64_t)kb << 10));
  const int k0 = kb * kColBlock;
#pragma unroll
  for (int s = 0; s < 4; ++s) B.gm[s] = *(gv4up)(grow + k0 + 32 * s);
#pragma unroll
  for (int j = 0; j < 4 * NC; ++j) (&B.b[0][0])[j] = *(gv8hp)(xrow[j] + k0);
}

// The last, partial block: lim = M - 128 kb < 128 entries exist; chunks past
// them are zero (not read).  xrow[j] already includes the lane's chunk, 8 *
// (lane % 16) entries.
template <int NC>
__device__ inline void load_block_tail(Block<NC, true>& B, const char* sq,
                                       const half_t* const (&xrow)[4 * NC], const half_t* grow,
                                       int kb, int lim, int g, int chunk) {
  B.a = *(gv4up)(sq + ((int64_t)kb << 10));
  const int k0 = kb * kColBlock;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bool ok = 32 * s + 8 * g < lim;
    B.gm[s] = ok ? *(gv4up)(grow + k0 + 32 * s) : v4u{0u, 0u, 0u, 0u};
  }
  const bool ok = 8 * chunk < lim;
#pragma unroll
  for (int j = 0; j < 4 * NC; ++j) (&B.b[0][0])[j] = ok ? *(gv8hp)(xrow[j] + k0) : v8h{};
}

// Row-chunk order -> operand order through the wave's LDS area: row r of
// the block is 256 bytes, its chunk c stored at position c ^ (r % 16), so
// the 8 or 16 lanes an LDS pass serves hit distinct banks on both sides.
// wr[j] / rd[s*NC + c] are the lane's byte offsets (loop invariant).
template <int NC>
__device__ inline void x_to_operand(Block<NC, true>& B, char* area, const int (&wr)[4 * NC],
                                    const int (&rd)[4 * NC]) {
#pragma unroll
  for (int j = 0; j < 4 * NC; ++j) *(v8h*)(area + wr[j]) = (&B.b[0][0])[j];
#pragma unroll
  for (int j = 0; j < 4 * NC; ++j) (&B.b[0][0])[j] = *(const v8h*)(area + rd[j]);
}

template <int NC, bool XIN>
__device__ inline void mma_block(v4f (&acc)[4][NC], const Block<NC, XIN>& B, uint32_t msk,
                                 uint32_t one) {
  auto step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    v8h a[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      a[h] = XIN ? expand_step_gamma<s>(B.a[h], msk, B.gm[XIN ? s : 0])
                 : expand_step_f16<s>(B.a[h], msk, one);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < 4; ++h)
        acc[h][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[h], B.b[s][c], acc[h][c], 0, 0, 0);
  };
  step(std::integral_constant<int, 0>{});
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 3>{});
}

// Half offset of entry (t, k) in one term's operand tiles.
__device__ inline int64_t tile_off(int t, int k, int nkb) {
  const int kk = k & 127;
  return ((int64_t)(t >> 4) * nkb + (k >> 7)) * 2048 + (kk >> 5) * 512 +
         (16 * ((kk >> 3) & 3) + (t & 15)) * 8 + (kk & 7);
}

struct PrepVParams {
  const half_t* x;
  int64_t ldx;
  int32_t T, M, ell, nkb, multi, num_adapters;
  int64_t n_units;  // ell * ceil(T/16) * nkb
  const half_t* gamma;
  const int32_t* ids;
  const half_t* const* gammas;
  half_t* v;
  int64_t v_term;
  // multi-adapter column blocks, built by the extra workgroup 0 (none when
  // seg_cbl is null)
  ColBlock* seg_cbl;
  WsHeader* seg_hdr;
  int32_t seg_chunk;
};

// v_i = fp16(gamma_i * x) in operand tiles, one wave per (term, 16-token
// tile, 128-block): lane 16g + c16 writes the 8 entries 32s + 8g .. of token
// c16 for each step s (1 KB contiguous per step).  Entries past M, tokens
// past T and tokens whose adapter id is out of range are zero.  One fp16
// rounding of the exact product.
template <bool MULTI>
__device__ inline void prep_v_block(const PrepVParams& p, int blk) {
  const int lane = threadIdx.x & 63;
  // unit counts fit 32 bits (the workspace bounds them; the host checks)
  const int u = blk * 4 + (threadIdx.x >> 6);
  if (u >= (int)p.n_units) return;  // uniform per wave
  const int r = u / p.nkb, kb = u - r * p.nkb;
  const int ntt = (p.T + 15) >> 4;
  const int i = r / ntt, tt = r - i * ntt;
  const int g = lane >> 4, c16 = lane & 15;
  const int t = tt * 16 + c16;
  const half_t* gam = nullptr;
  if (t < p.T) {
    if (MULTI) {
      const int32_t ad = norm_id(p.ids[t], p.num_adapters);
      if (ad >= 0) gam = p.gammas[ad];
    } else {
      gam = p.gamma;
    }
  }
  half_t* out = p.v + i * p.v_term + ((int64_t)tt * p.nkb + kb) * 2048 + lane * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k = kb * kColBlock + 32 * s + 8 * g;
    v8h o = {};
    if (gam != nullptr) {
      const half_t* xr = p.x + (int64_t)t * p.ldx + k;
      const half_t* gr = gam + (int64_t)i * p.M + k;
      if (k + 8 <= p.M) {
        const v8h xv = *(gv8hp)xr;
        v8h gv;
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] = gr[e];
        o = xv * gv;
      } else {
        for (int e = 0; e < 8; ++e)
          if (k + e < p.M) o[e] = xr[e] * gr[e];
      }
    }
    *(v8h*)(out + s * 512) = o;
  }
}

template <bool MULTI>
__global__ __launch_bounds__(256) void k_prep_v(PrepVParams p) {
  if (MULTI && p.seg_cbl != nullptr && blockIdx.x == 0) {
    segment_ids(p.ids, p.T, p.num_adapters, p.seg_chunk, p.seg_cbl, p.seg_hdr);
    return;
  }
  prep_v_block<MULTI>(p, (int)blockIdx.x - (MULTI && p.seg_cbl != nullptr ? 1 : 0));
}

// Two independent one-adapter tile builds in one launch: workgroups [0, n0)
// build p0's tiles, the rest p1's.
__global__ __launch_bounds__(256) void k_prep_v2(PrepVParams p0, PrepVParams p1, int32_t n0) {
  const int b = (int)blockIdx.x;
  if (b < n0)
    prep_v_block<false>(p0, b);
  else
    prep_v_block<false>(p1, b - n0);
}

// Several adapters: the first column block of a workgroup and, for up to
// kLdsAdapters adapters, the factor pointer tables (B1, B2, alpha, beta) are
// requested together with the column-block count at the start; the tables
// go to LDS, so the first item waits for one memory round trip instead of
// three (count, then block, then pointers).  Workgroup-wide.
constexpr int kLdsAdapters = 256;
template <int CAP>
struct FactorTab {
  const void* ptr[CAP][4];
};
__device__ inline ColBlock prefetch_multi(const GemmParams& p, int first,
                                          FactorTab<kLdsAdapters>& tab) {
  const int cb0 = first / p.n_rg;
  const ColBlock c = p.cbl[cb0 < p.cb_cap ? cb0 : p.cb_cap - 1];
  if (p.num_adapters <= kLdsAdapters) {
    for (int e = threadIdx.x; e < p.num_adapters; e += blockDim.x) {
      tab.ptr[e][0] = p.B1s[e];
      tab.ptr[e][1] = p.B2s[e];
      tab.ptr[e][2] = p.alphas[e];
      tab.ptr[e][3] = p.betas[e];
    }
  }
  __syncthreads();
  return c;
}
__device__ inline void factors_of(const GemmParams& p, const FactorTab<kLdsAdapters>& tab, int ad,
                                  Factors& f) {
  if (p.num_adapters <= kLdsAdapters) {
    f.B1 = (const uint32_t*)tab.ptr[ad][0];
    f.B2 = (const uint32_t*)tab.ptr[ad][1];
    f.alpha = (const half_t*)tab.ptr[ad][2];
    f.beta = (const half_t*)tab.ptr[ad][3];
  } else {
    f.B1 = p.B1s[ad];
    f.B2 = p.B2s[ad];
    f.alpha = p.alphas[ad];
    f.beta = p.betas[ad];
  }
}

template <int STAGE, int NC, bool SPLITK, bool MULTI, bool XIN, int NWV, bool GROUP>
__global__ __launch_bounds__(64 * NWV) void k_gemm(GemmParams p) {
  static_assert(!XIN || (STAGE == 1 && !MULTI), "x is read in place by single-adapter stage 1");
  static_assert(!GROUP || !MULTI, "grouped layers take the single-adapter stages");
  static_assert(NWV == 4 || (SPLITK && NC == 2 && NWV == 8), "8 waves only split a reduction");
  constexpr int D = 2;  // operand buffers per wave (deeper rings measured slower)
  constexpr int TPW = 4 * NC / NWV;  // SPLITK: output tiles each wave finishes
  __shared__ v4f red[SPLITK ? NWV : 1][SPLITK ? 4 * NC : 1][64];
  // x staging (XIN): 16*NC rows of 256 bytes per wave
  __shared__ v8h xst[XIN ? NWV : 1][XIN ? 16 * NC * 16 : 1];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const uint32_t one = p.one16;
  // item counts fit 32 bits (the workspace bounds T * R; the host checks)
  const int n_cb = MULTI ? p.hdr->n_colblocks : p.n_cb_host;
  const int n_per = n_cb * p.n_rg;  // items of one layer
  const int n_items = GROUP ? n_per * p.group : n_per;
  // consecutive items share a column block; with the remap the items of one
  // XCD (workgroups b, b+8, ...) are consecutive, so they share operand
  // tiles in that XCD's L2
  const int b = blockIdx.x;
  const int first = p.xcd_remap ? (b & 7) * (p.grid >> 3) + (b >> 3) : b;
  __shared__ FactorTab<MULTI ? kLdsAdapters : 1> ftab;
  ColBlock cb_first{};
  if constexpr (MULTI) cb_first = prefetch_multi(p, first, ftab);

  for (int it = first; it < n_items; it += p.grid) {
    int layer = 0, itl = it;
    if constexpr (GROUP) {
      layer = it / n_per;
      itl = it - layer * n_per;
    }
    const int cb = itl / p.n_rg, rg = itl - cb * p.n_rg;
    half_t* const zl = (half_t*)((char*)p.z + (GROUP ? layer * p.layer_ws : 0));
    const half_t* const ol = (const half_t*)((const char*)p.opnd + (GROUP ? layer * p.layer_ws : 0));
    void* const yl = (char*)p.y + (GROUP ? layer * p.y_layer_bytes : 0);
    int t0, t1, ad;
    Factors f;
    if constexpr (MULTI) {
      const ColBlock cbk = it == first ? cb_first : p.cbl[cb];
      t0 = cbk.t0;
      t1 = cbk.t1;
      ad = cbk.adapter;
      if constexpr (MULTI)
        if (ad >= 0) factors_of(p, ftab, ad, f);
    } else {
      t0 = cb * 16 * NC;
      t1 = t0 + 16 * NC < p.T ? t0 + 16 * NC : p.T;
      ad = 0;
      f = GROUP ? p.grp[layer] : p.single;
    }
    const int q = SPLITK ? rg : 4 * rg + wv;  // row quad of this wave
    const int row_lo = (SPLITK ? rg : 4 * rg) * kQuad * kRowTile;
    const int row_hi = min(p.rows, row_lo + (SPLITK ? 1 : 4) * kQuad * kRowTile);
    if (ad < 0) {
      // tokens whose adapter id is out of range: y = 0 (or unchanged); their
      // z is never read (stage 2 skips the same column blocks)
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
    // this wave's 128-blocks: wv, wv+NWV, ... (SPLITK) or all of them; with
    // x read in place a partial last block is taken apart from the others
    const int nfull = XIN ? p.K / kColBlock : p.nkb;
    const int kb0 = SPLITK ? wv : 0, kst = SPLITK ? NWV : 1;
    const int nkw = SPLITK ? (nfull - wv + NWV - 1) / NWV : nfull;
    const bool run = active && nkw > 0;
    const bool tail = XIN && active && nfull < p.nkb && (!SPLITK || nfull % NWV == wv);
    float ys[SPLITK ? TPW : 4 * NC][4];  // stage 2: running sum over the terms

    for (int i = 0; i < p.ell; ++i) {
      // row scales of this wave's quad (lane L: row 64q + L), loaded first
      // and kept as loaded (converting here would wait for the load); lanes
      // fetch the ones they need with a cross-lane read at the end
      const int srow = q * kQuad * kRowTile + lane;
      half_t sclh = (half_t)1.0f;  // stage 3 scales nothing
      if constexpr (STAGE != 3) {
        const half_t* sv = (STAGE == 1 ? f.beta : f.alpha) + (int64_t)i * p.rows;
        sclh = sv[min(srow, p.rows - 1)];
      }
      // operand rows: tile rows of v / z, or (XIN) lane's chunk of x row
      // L/16 + 4j of the column block
      const half_t* orow[XIN ? 4 * NC : NC];
      if constexpr (XIN) {
#pragma unroll
        for (int j = 0; j < 4 * NC; ++j) {
          const int t = min(t0 + (lane >> 4) + 4 * j, t1 - 1);
          orow[j] = p.x + (int64_t)t * p.ldx + 8 * c16;
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int t = min(t0 + 16 * c + c16, t1 - 1);
          orow[c] = ol + i * p.opnd_term + (int64_t)(t >> 4) * p.opnd_nkb * 2048 +
                    (16 * g + (t & 15)) * 8;
        }
      }
      const half_t* grow = XIN ? f.gamma + (int64_t)i * p.K + 8 * g : nullptr;
      // XIN: LDS byte offsets of the lane's chunk writes (row L/16 + 4j,
      // chunk L%16) and operand reads (step s, token column c: row 16c + c16,
      // chunk 4s + g)
      int wr[XIN ? 4 * NC : 1], rd[XIN ? 4 * NC : 1];
      if constexpr (XIN) {
#pragma unroll
        for (int j = 0; j < 4 * NC; ++j) {
          const int r = (lane >> 4) + 4 * j;
          wr[j] = r * 256 + ((c16 ^ (r & 15)) << 4);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int c = 0; c < NC; ++c)
            rd[s * NC + c] = (16 * c + c16) * 256 + (((4 * s + g) ^ c16) << 4);
      }
      char* xarea = (char*)&xst[XIN ? wv : 0][0];

      v4f acc[4][NC];
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[h][c] = v4f{0.f, 0.f, 0.f, 0.f};

      if (run) {
        // Operands of the next D-1 blocks are in flight while one is
        // consumed: D buffers with fixed roles (the loop is unrolled by D),
        // refilled right after their last use.  Every step issues the same
        // loads (clamped at the end), so each in-order wait covers exactly
        // the buffer about to be used.
        auto kb_of = [&](int j) { return kb0 + min(j, nkw - 1) * kst; };
        auto load = [&](Block<NC, XIN>& B, int kb) {
          if constexpr (XIN)
            load_block<NC>(B, sq, orow, grow, kb);
          else
            load_block<NC>(B, sq, orow, kb);
        };
        Block<NC, XIN> buf[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load(buf[d], kb_of(d));
        for (int j = 0; j < nkw; j += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            if (j + d < nkw) {
              if constexpr (XIN) x_to_operand<NC>(buf[d], xarea, wr, rd);
              mma_block<NC, XIN>(acc, buf[d], p.msk16, one);
            }
            __builtin_amdgcn_sched_barrier(0);
            load(buf[d], kb_of(j + d + D));
          }
        }
      }
      if constexpr (XIN) {
        if (tail) {
          Block<NC, true> B;
          load_block_tail<NC>(B, sq, orow, grow, nfull, p.K - nfull * kColBlock, g, c16);
          x_to_operand<NC>(B, xarea, wr, rd);
          mma_block<NC, true>(acc, B, p.msk16, one);
        }
      }

      if (SPLITK) {
        // fixed-order sum of the waves' partial tiles; wave w finishes
        // tiles w*TPW .. w*TPW + TPW-1 (tile = h*NC + c)
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int c = 0; c < NC; ++c) red[wv][h * NC + c][lane] = acc[h][c];
        __syncthreads();
      }
      if (active) {
        const float scl = srow < p.rows ? (float)sclh : 0.0f;
        constexpr int NE = SPLITK ? TPW : 4 * NC;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int tile = SPLITK ? wv * TPW + e : e, h = tile / NC, c = tile % NC;
          v4f sum;
          if (SPLITK) {
            sum = red[0][tile][lane];
#pragma unroll
            for (int w = 1; w < NWV; ++w) sum += red[w][tile][lane];
          } else {
            sum = acc[h][c];
          }
          const int rl = h * kRowTile + 4 * g;  // quad-local row of v = 0
          const int r0 = q * kQuad * kRowTile + rl;
          const int t = t0 + 16 * c + c16;
          float sc[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[v] = __shfl(scl, rl + v, 64);
          if (STAGE == 1) {
            // rows r0..r0+3 share one 8-entry chunk of the z tile; rows past
            // R get scale 0, so the chunk is written whole
            if (t < t1)
              *(v4h*)(zl + i * p.z_term + tile_off(t, r0, p.z_nkb)) =
                  v4h{(half_t)(sum[0] * sc[0]), (half_t)(sum[1] * sc[1]),
                      (half_t)(sum[2] * sc[2]), (half_t)(sum[3] * sc[3])};
          } else if (STAGE == 3) {
            if (t < t1 && r0 < p.rows) {
              const float o[4] = {sum[0], sum[1], sum[2], sum[3]};
              store4((float*)yl + i * p.y_term, p.ldy, true, t, r0, p.rows, o);
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
                load4(yl, p.ldy, p.y_f32, t, r0, p.rows, old);
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] += old[v];
              }
              store4(yl, p.ldy, p.y_f32, t, r0, p.rows, o);
            }
          }
        }
        // stage 1: when the row quads stop half way through the last 128-row
        // block of z, the quad before the gap zeroes the rest of that block
        if (STAGE == 1 && q == p.nq - 1 && (p.nq & 1) && (!SPLITK || wv == 0)) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int t = t0 + 16 * c + c16;
            if (t < t1)
#pragma unroll
              for (int h = 0; h < 4; ++h)
                *(v4h*)(zl + i * p.z_term + tile_off(t, p.nq * 64 + h * 16 + 4 * g, p.z_nkb)) =
                    v4h{};
          }
        }
      }
      if (SPLITK) __syncthreads();
    }
  }
}

// Stage 2 when every term's whole reduction fits in registers (ell *
// ceil(R/128) <= KT = 2: short ranks).  A work item is a column block of 32
// tokens and kKregQG row quads.  The token operands of every (term, block),
// the sign words of the wave's quads (w, w+4, ... of the group) and the
// item's alpha rows (into LDS) are requested together at the start, so an
// item waits for one memory round trip.  alpha_i is folded into the expanded sign
// operand: alpha_i[row] * (+-1) is exact in fp16 (the sign bits are XORed
// into alpha's), so one fp32 accumulator per tile sums every term's products
// and the epilogue only stores.
constexpr int64_t kComputeUnits = 256;  // MI355X
constexpr int kKregQG = 16;              // row quads per work item
constexpr int kKregQPW = kKregQG / 4;     // per wave

template <int s>
__device__ inline v8h expand_step_scaled(uint32_t w, uint32_t msk, uint32_t apair) {
  const uint32_t U = w << (7 - s), V = w << (3 - s);
  v4u o;
  o[0] = (__builtin_amdgcn_perm(V, U, 0x040C000Cu) & msk) ^ apair;
  o[1] = (__builtin_amdgcn_perm(V, U, 0x050C010Cu) & msk) ^ apair;
  o[2] = (__builtin_amdgcn_perm(V, U, 0x060C020Cu) & msk) ^ apair;
  o[3] = (__builtin_amdgcn_perm(V, U, 0x070C030Cu) & msk) ^ apair;
  return __builtin_bit_cast(v8h, o);
}

template <int KT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_kreg(GemmParams p) {
  constexpr int NC = 2;
  static_assert(NC == 2, "the second token tile is optional");
  __shared__ half_t sa[KT * kKregQG * kQuad * kRowTile];  // alpha rows of the item
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int n_cb = p.multi ? p.hdr->n_colblocks : p.n_cb_host;
  const int n_items = n_cb * p.n_rg;  // fits 32 bits (the host checks)
  const int nkb = p.nkb, ell = p.ell, rows = p.rows;

  __shared__ FactorTab<kLdsAdapters> ftab;
  ColBlock cb_first{};
  if (p.multi) cb_first = prefetch_multi(p, blockIdx.x, ftab);
  for (int it = blockIdx.x; it < n_items; it += p.grid) {
    const int cb = it / p.n_rg, rg = it - cb * p.n_rg;
    int t0, t1, ad;
    Factors f;
    if (p.multi) {
      const ColBlock cbk = it == (int)blockIdx.x ? cb_first : p.cbl[cb];
      t0 = cbk.t0;
      t1 = cbk.t1;
      ad = cbk.adapter;
      if (ad >= 0) factors_of(p, ftab, ad, f);
    } else {
      t0 = cb * 16 * NC;
      t1 = t0 + 16 * NC < p.T ? t0 + 16 * NC : p.T;
      ad = 0;
      f = p.single;
    }
    const int qlo = rg * kKregQG, qhi = min(p.nq, qlo + kKregQG);
    if (ad < 0) {
      // tokens whose adapter id is out of range: y = 0 (or unchanged)
      if (!p.accumulate) {
        const int r_lo = qlo * kQuad * kRowTile, nr = min(rows, qhi * kQuad * kRowTile) - r_lo;
        for (int e = threadIdx.x; e < (t1 - t0) * nr; e += blockDim.x) {
          const int64_t t = t0 + e / nr, r = r_lo + e % nr;
          if (p.y_f32)
            ((float*)p.y)[t * p.ldy + r] = 0.0f;
          else
            ((half_t*)p.y)[t * p.ldy + r] = (half_t)0.0f;
        }
      }
      continue;
    }
    // token operands of every (term, block): tb = term * nkb + block
    v8h b[KT][4][NC];
#pragma unroll
    for (int tb = 0; tb < KT; ++tb) {
      const int i = tb / nkb, kb = tb - i * nkb;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int t = min(t0 + 16 * c + c16, t1 - 1);
        const half_t* orow = p.opnd + (int64_t)i * p.opnd_term +
                             (int64_t)(t >> 4) * p.opnd_nkb * 2048 + (16 * g + (t & 15)) * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          b[tb][s][c] = i < ell ? *(gv8hp)(orow + (int64_t)kb * 2048 + s * 512) : v8h{};
      }
    }
    const bool two_tiles = t1 - t0 > 16;
    // sign words of this wave's quads (q = qlo + wv + 4j; one v4u per
    // block) requested together, and the item's alpha rows staged in LDS
    const char* sgn = (const char*)f.B1 + lane * 16;
    v4u w[kKregQPW][KT];
#pragma unroll
    for (int jq = 0; jq < kKregQPW; ++jq) {
      const int q = qlo + wv + 4 * jq;
#pragma unroll
      for (int kb = 0; kb < KT; ++kb)
        w[jq][kb] = (q < qhi && kb < nkb) ? *(gv4up)(sgn + (((int64_t)q * nkb + kb) << 10))
                                          : v4u{0u, 0u, 0u, 0u};
    }
    constexpr int kRowsItem = kKregQG * kQuad * kRowTile;
    {
      constexpr int kPer = KT * kRowsItem / 256;
      half_t av[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = threadIdx.x + 256 * u;
        const int i = e / kRowsItem, r = qlo * kQuad * kRowTile + e - i * kRowsItem;
        av[u] = (i < ell && r < rows) ? f.alpha[(int64_t)i * rows + r] : (half_t)0.0f;
      }
      __syncthreads();  // the previous item's readers of sa are done
#pragma unroll
      for (int u = 0; u < kPer; ++u) sa[threadIdx.x + 256 * u] = av[u];
      __syncthreads();
    }
#pragma unroll
    for (int jq = 0; jq < kKregQPW; ++jq) {
      const int q = qlo + wv + 4 * jq;
      if (q >= qhi) break;
      // alpha pairs of this lane's rows (tile h, row c16) for every term
      uint32_t ap[KT][4];
#pragma unroll
      for (int i = 0; i < KT; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t ab = __builtin_bit_cast(
              uint16_t, sa[i * kRowsItem + (q - qlo) * kQuad * kRowTile + h * kRowTile + c16]);
          ap[i][h] = ab | (ab << 16);
        }
      v4f acc[4][NC];
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[h][c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tb = 0; tb < KT; ++tb) {
        const int i = tb / nkb, kb = tb - i * nkb;
        // steps wholly past the rank meet zero operands, and so do the
        // columns of a second token tile the block does not reach: both
        // are skipped (wave-uniform tests)
        const int kvalid = p.K - kb * kColBlock;
        if (i < ell) {
          auto step = [&](auto sc) {
            constexpr int st = decltype(sc)::value;
            if (32 * st >= kvalid) return;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const v8h a = expand_step_scaled<st>(w[jq][kb][h], p.msk16, ap[i][h]);
              acc[h][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[tb][st][0], acc[h][0], 0, 0, 0);
              if (two_tiles)
                acc[h][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[tb][st][1], acc[h][1], 0, 0, 0);
            }
          };
          step(std::integral_constant<int, 0>{});
          step(std::integral_constant<int, 1>{});
          step(std::integral_constant<int, 2>{});
          step(std::integral_constant<int, 3>{});
        }
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int t = t0 + 16 * c + c16;
          const int r0 = q * kQuad * kRowTile + h * kRowTile + 4 * g;
          if (t < t1 && r0 < rows) {
            float o[4] = {acc[h][c][0], acc[h][c][1], acc[h][c][2], acc[h][c][3]};
            if (p.accumulate) {
              float old[4];
              load4(p.y, p.ldy, p.y_f32, t, r0, rows, old);
#pragma unroll
              for (int v = 0; v < 4; ++v) o[v] += old[v];
            }
            store4(p.y, p.ldy, p.y_f32, t, r0, rows, o);
          }
        }
    }
  }
}

// Whether a single-adapter stage takes 64-token column blocks.
inline bool wide_blocks(const GemmParams& p) {
  return p.nkb >= 4 && cdiv(p.T, 64) * p.nq >= 512;
}

// Whether a split-reduction stage runs 8 waves per workgroup: single
// adapter, 32-token blocks and no more items than compute units.
inline bool eight_waves(const GemmParams& p) {
  return !p.multi && p.nkb >= 4 && !wide_blocks(p) && cdiv(p.T, 32) * p.nq <= kComputeUnits;
}

template <int STAGE, int NC, bool SPLITK, bool MULTI, bool XIN, bool GROUP>
hipError_t launch_k(const GemmParams& p, int64_t grid, bool wide, hipStream_t s) {
  if constexpr (SPLITK && !MULTI && NC == 2) {  // 64-token blocks would spill at 8 waves
    if (wide) {
      hipLaunchKernelGGL((k_gemm<STAGE, NC, SPLITK, MULTI, XIN, 8, GROUP>), dim3((unsigned)grid),
                         dim3(512), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((k_gemm<STAGE, NC, SPLITK, MULTI, XIN, 4, GROUP>), dim3((unsigned)grid),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int STAGE, int NC, bool SPLITK>
hipError_t launch_one(GemmParams p, hipStream_t s) {
  p.n_rg = SPLITK ? p.nq : (p.nq + 3) / 4;
  const int64_t items = (int64_t)p.n_cb_host * p.n_rg * (p.group > 1 ? p.group : 1);
  if (items > INT32_MAX) return hipErrorInvalidValue;
  int64_t grid = items;
  if (p.multi && grid > 8192) grid = 8192;
  // with several adapters the item count is known only on the device, so
  // consecutive items cannot be mapped to one XCD
  p.xcd_remap = (!p.multi && grid == items && items % 8 == 0) ? 1 : 0;
  p.grid = (int32_t)grid;
  // the wave count follows one layer's items, as for a single call
  const bool wide = eight_waves(p);
  if (p.multi) return launch_k<STAGE, NC, SPLITK, true, false, false>(p, grid, false, s);
  if (p.group > 1) {
    if constexpr (STAGE >= 2) return launch_k<STAGE, NC, SPLITK, false, false, true>(p, grid, wide, s);
    if constexpr (STAGE == 1 && NC == 2) {
      if (p.x != nullptr) return launch_k<1, NC, SPLITK, false, true, true>(p, grid, wide, s);
    }
    return hipErrorNotSupported;
  }
  if constexpr (STAGE == 1 && NC == 2) {
    if (p.x != nullptr) return launch_k<1, NC, SPLITK, false, true, false>(p, grid, wide, s);
  }
  return launch_k<STAGE, NC, SPLITK, false, false, false>(p, grid, wide, s);
}

template <int STAGE>
hipError_t launch_stage(GemmParams p, hipStream_t s) {
  if (STAGE == 2 && (int64_t)p.ell * p.nkb <= 2) {
    // short reduction: operands held in registers, row quads streamed
    if (!p.multi) p.n_cb_host = (int32_t)cdiv(p.T, 32);
    p.n_rg = (int32_t)cdiv(p.nq, kKregQG);
    int64_t grid = (int64_t)p.n_cb_host * p.n_rg;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    if (grid > 8192) grid = 8192;
    p.grid = (int32_t)grid;
    hipLaunchKernelGGL((k_gemm_kreg<2>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  const bool split = p.nkb >= 4;
  if (p.multi) {
    return split ? launch_one<STAGE, 2, true>(p, s) : launch_one<STAGE, 2, false>(p, s);
  }
  if (wide_blocks(p)) {
    p.n_cb_host = (int32_t)cdiv(p.T, 64);
    return launch_one<STAGE, 4, true>(p, s);
  }
  p.n_cb_host = (int32_t)cdiv(p.T, 32);
  return split ? launch_one<STAGE, 2, true>(p, s) : launch_one<STAGE, 2, false>(p, s);
}

}  // namespace

hipError_t launch_tiles_f16_pair(const TilesF16& a, const TilesF16& b, int64_t T, int32_t ell,
                                 hipStream_t s) {
  PrepVParams pv[2]{};
  int64_t blocks[2];
  for (int j = 0; j < 2; ++j) {
    const TilesF16& t = j == 0 ? a : b;
    PrepVParams& q = pv[j];
    q.x = t.src;
    q.ldx = t.ld;
    q.T = (int32_t)T;
    q.M = (int32_t)t.K;
    q.ell = ell;
    q.nkb = (int32_t)cdiv(t.K, kColBlock);
    q.n_units = (int64_t)ell * cdiv(T, 16) * q.nkb;
    q.gamma = t.scale;
    q.v = t.out;
    q.v_term = zt_term_halfs(t.K, T);
    if (q.n_units > INT32_MAX - 4) return hipErrorInvalidValue;
    blocks[j] = cdiv(q.n_units, 4);
  }
  if (blocks[0] + blocks[1] > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prep_v2, dim3((unsigned)(blocks[0] + blocks[1])), dim3(256), 0, s, pv[0],
                     pv[1], (int32_t)blocks[0]);
  return hipGetLastError();
}

namespace {
GemmParams sign_product_params(int64_t rows, int64_t K, int32_t ell, int64_t T, float* out,
                               int64_t ldo) {
  GemmParams p{};
  p.rows = (int32_t)rows;
  p.K = (int32_t)K;
  p.T = (int32_t)T;
  p.ell = ell;
  p.nq = (int32_t)cdiv(rows, kRowTile * kQuad);
  p.nkb = (int32_t)cdiv(K, kColBlock);
  p.msk16 = 0x80008000u;
  p.one16 = 0x3C003C00u;
  p.y_f32 = 1;
  p.y = out;
  p.ldy = ldo;
  p.y_term = T * ldo;
  p.opnd_term = zt_term_halfs(K, T);
  p.opnd_nkb = p.nkb;
  return p;
}
}  // namespace

hipError_t launch_sign_product(const uint32_t* S, int64_t rows, int64_t K, int32_t ell, int64_t T,
                               const half_t* tiles, float* out, int64_t ldo, hipStream_t s) {
  GemmParams p = sign_product_params(rows, K, ell, T, out, ldo);
  p.single.B1 = S;
  p.opnd = tiles;
  return launch_stage<3>(p, s);
}

hipError_t launch_sign_product_pair(const uint32_t* S0, const uint32_t* S1, int64_t rows,
                                    int64_t K, int32_t ell, int64_t T, const half_t* tiles0,
                                    const half_t* tiles1, float* out0, float* out1, int64_t ldo,
                                    hipStream_t s) {
  GemmParams p = sign_product_params(rows, K, ell, T, out0, ldo);
  // the second product as layer 1 of a grouped launch: its operand tiles
  // and its output at fixed byte offsets from the first's
  p.group = 2;
  p.grp[0].B1 = S0;
  p.grp[1].B1 = S1;
  p.opnd = tiles0;
  p.layer_ws = (int64_t)((const char*)tiles1 - (const char*)tiles0);
  p.y_layer_bytes = (int64_t)((const char*)out1 - (const char*)out0);
  return launch_stage<3>(p, s);
}

hipError_t launch_gemm(const ForwardArgs& a, hipStream_t s) {
  // several adapters of short rank: token tiles served adapter by adapter
  if (ma_short_fits(a)) return launch_ma_short(a, s);
  // one adapter: the shared-token-tile stages (dbf_tile.hip); grouped
  // layers then run one by one through the same stages, so each layer's
  // result is that of dbf_forward on it
  if (!a.multi && tile_path_fits(a)) {
    if (a.group > 1) return hipErrorNotSupported;
    return launch_tile_forward(a, s);
  }
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  char* ws = (char*)a.ws;
  GemmParams p{};
  if (a.multi) {
    // column blocks of at most kGemmChunk tokens of one adapter (built by
    // the prep launch)
    // the grid follows an estimate (one partial block per adapter plus
    // full blocks); workgroups loop over any further blocks
    int64_t n_cb = (int64_t)a.num_adapters + cdiv(a.T, kGemmChunk);
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
  p.y = a.y;
  p.ldy = a.ldy;
  p.single = a.single;
  p.cbl = (const ColBlock*)(ws + L.cbl);
  p.hdr = (const WsHeader*)ws;
  p.cb_cap = (int32_t)max_colblocks(a.T);
  p.num_adapters = a.multi ? a.num_adapters : 0;
  p.B1s = a.B1s;
  p.B2s = a.B2s;
  p.alphas = a.alphas;
  p.betas = a.betas;
  half_t* vt = (half_t*)(ws + L.v);
  half_t* zt = (half_t*)(ws + L.z);

  GemmParams p1 = p, p2 = p;
  p1.rows = (int32_t)a.R;
  p1.K = (int32_t)a.M;
  p1.nq = (int32_t)cdiv(a.R, kRowTile * kQuad);
  p1.nkb = (int32_t)cdiv(a.M, kColBlock);
  p1.opnd = vt;
  p1.opnd_term = zt_term_halfs(a.M, a.T);
  p1.opnd_nkb = p1.nkb;
  p1.z = zt;
  p1.z_term = zt_term_halfs(a.R, a.T);
  p1.z_nkb = (int32_t)cdiv(a.R, kColBlock);
  p2.rows = (int32_t)a.N;
  p2.K = (int32_t)a.R;
  p2.nq = (int32_t)cdiv(a.N, kRowTile * kQuad);
  p2.nkb = (int32_t)cdiv(a.R, kColBlock);
  p2.opnd = zt;
  p2.opnd_term = zt_term_halfs(a.R, a.T);
  p2.opnd_nkb = p2.nkb;
  // Stage 1 reads x in place when every 8-entry chunk of x and gamma is a
  // whole aligned 16-byte load (x and ldx are checked by the caller), with
  // 32-token column blocks (64 would not fit the registers), and when each
  // wave has at most 8 blocks of the reduction: passing x through LDS costs
  // about 0.3 us per block, the prep launch it replaces about 3 us.
  const int nwv1 = eight_waves(p1) ? 8 : 4;
  const bool xin = !a.multi && a.M % 8 == 0 && (((uintptr_t)a.single.gamma) & 15u) == 0 &&
                   !wide_blocks(p1) && cdiv(p1.nkb, nwv1) <= 8;
  if (xin) {
    p1.x = a.x;
    p1.ldx = a.ldx;
  }
  if (a.group > 1) {
    // one launch per stage for every layer: stage 1 reads x in place for all
    // of them and stage 2 is not the short-rank register kernel; otherwise the
    // caller runs the layers one by one (nothing has been launched)
    bool ok = xin && (int64_t)a.ell * p2.nkb > 2;
    for (int j = 0; j < a.group; ++j) ok = ok && (((uintptr_t)a.grp[j].gamma) & 15u) == 0;
    if (!ok) return hipErrorNotSupported;
    for (GemmParams* q : {&p1, &p2}) {
      q->group = a.group;
      q->layer_ws = (int64_t)a.layer_ws;
      q->y_layer_bytes = a.y_layer_bytes;
      for (int j = 0; j < a.group; ++j) q->grp[j] = a.grp[j];
    }
    if (a.phases & 2) {
      const hipError_t e = launch_stage<1>(p1, s);
      if (e != hipSuccess) return e;
    }
    return (a.phases & 4) ? launch_stage<2>(p2, s) : hipSuccess;
  }

  if ((a.phases & 1) && !xin) {
    PrepVParams pv{};
    pv.x = a.x;
    pv.ldx = a.ldx;
    pv.T = (int32_t)a.T;
    pv.M = (int32_t)a.M;
    pv.ell = a.ell;
    pv.nkb = p1.nkb;
    pv.multi = a.multi;
    pv.num_adapters = a.num_adapters;
    pv.n_units = (int64_t)a.ell * cdiv(a.T, 16) * p1.nkb;
    pv.gamma = a.single.gamma;
    pv.ids = a.ids;
    pv.gammas = a.gammas;
    pv.v = vt;
    pv.v_term = p1.opnd_term;
    if (a.multi) {
      pv.seg_cbl = (ColBlock*)(ws + L.cbl);
      pv.seg_hdr = (WsHeader*)ws;
      pv.seg_chunk = kGemmChunk;
    }
    const int64_t grid = cdiv(pv.n_units, 4) + (a.multi ? 1 : 0);
    if (pv.n_units > INT32_MAX - 4) return hipErrorInvalidValue;
    if (a.multi)
      hipLaunchKernelGGL(k_prep_v<true>, dim3((unsigned)grid), dim3(256), 0, s, pv);
    else
      hipLaunchKernelGGL(k_prep_v<false>, dim3((unsigned)grid), dim3(256), 0, s, pv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.phases & 2) {
    const hipError_t e = launch_stage<1>(p1, s);
    if (e != hipSuccess) return e;
  }
  return (a.phases & 4) ? launch_stage<2>(p2, s) : hipSuccess;
}

}  // namespace dbf
