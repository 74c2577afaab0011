// Several adapters at large T with a short rank (R <= 64, at most two terms):
// token tiles of 16 served adapter by adapter, one launch per stage.
//
// The batch is the serving case of the LoRDBA summary (section 1: many
// unmerged adapters in one batch, each token with its own adapter) and each
// token's product is the DBF summary's inference computation (section 2:
// two sign products with the scalings between them), with the terms of the
// LoRDBA sum (section 2, "Nucleo de Inferencia") added in order.
//
// A one-workgroup launch cuts the ids into column blocks: runs of at most
// 16 tokens of one adapter (any order of ids is accepted; sorted ids give
// about T/16 + A blocks).  A block's tokens are one MFMA column each; the
// other columns (stage 1: whatever the LDS area holds, since only the
// block's x rows are requested; stage 2: zero) are computed and not stored.
//   stage 1 (R <= 64 rows: one row quad), 8 waves: wave w accumulates the
//     128-blocks w, w + 8, ... of the reduction over M; each wave requests
//     all of a chunk's x rows straight into its own LDS area (256
//     contiguous bytes per 16 lanes) and its sign words before its first
//     MFMA, with gamma_i in LDS; B = fp16(x * gamma_i), one rounding of the exact
//     product, as on the single-adapter path.  The 8 partial tiles are
//     summed in wave order through LDS, scaled by beta_i in fp32 and rounded
//     once to fp16: z [ell][T][ldz] in the workspace.  One workgroup per
//     block.
//   stage 2, 4 waves per (block, 8 row quads of the N outputs): the
//     reduction over R is at most two MFMA steps per term; each term's tile
//     is scaled by alpha_i in fp32 and the terms are added in ascending i;
//     the tile goes through LDS so that each token's 64 outputs leave as one
//     128-byte (fp16) or 256-byte (fp32) run.
// Ids outside [0, A) write y = 0 (unchanged under ACCUMULATE).
#include "dbf_device.h"
#include "dbf_launch.h"

namespace dbf {

namespace {

constexpr int kMaTok = 16;           // tokens per column block
constexpr int kMaW1 = 8;             // stage-1 waves per workgroup
constexpr int kMaBlk = 4;            // 128-blocks per wave per chunk of stage 1
constexpr int kMaW2 = 4;             // stage-2 waves per workgroup
constexpr int kMaQw = 2;             // stage-2 row quads per wave
constexpr int kMaMaxEll = 2;         // terms
constexpr int kMaGamHalfs = 8704;    // LDS halfs for gamma_i of every term, zero-padded
constexpr int kMaStage = (kMaGamHalfs / 8 + 64 * kMaW1 - 1) / (64 * kMaW1);  // chunks per thread

struct MaParams {
  const half_t* x;
  int64_t ldx;
  const int32_t* ids;
  int32_t num_adapters;
  const uint32_t* const* B1s;
  const uint32_t* const* B2s;
  const half_t* const* alphas;
  const half_t* const* betas;
  const half_t* const* gammas;
  half_t* z;  // workspace: z [ell][T][ldz]
  int32_t ldz;
  const ColBlock* cbl;  // workspace: the column blocks and their count
  const WsHeader* hdr;
  ColBlock* cbl_w;      // (the same, written by the segmentation)
  WsHeader* hdr_w;
  int32_t n_cb_est;     // stage-1 workgroups (stage 2: times nch2)
  void* y;
  int64_t ldy;
  int32_t y_f32, accumulate;
  int32_t N, R, M, T, ell;
  int32_t nkb1;  // 128-blocks of the stage-1 reduction
  int32_t nq2;   // row quads of stage 2
  int32_t nch2;  // stage-2 workgroups per tile
  uint32_t nib_mask, nib_one;
};

typedef const DBF_GLOBAL half_t* ghp;
// Reads through the constant address space with wave-uniform addresses are
// scalar loads: waiting for them does not wait for the vector requests in
// flight (the x rows of stage 1).  The block list, the count and the factor
// pointer tables are not written during a launch that reads them.
typedef const __attribute__((address_space(4))) int32_t* cip;
typedef const __attribute__((address_space(4))) uint64_t* cu64p;

// Entry a of a pointer table (a wave-uniform): one scalar load.
template <class P>
__device__ inline P table_ptr(const void* tab, int32_t a) {
  return (P)(uintptr_t)((cu64p)tab)[a];
}

// The column blocks (runs of at most 16 tokens of one adapter, from the
// segmentation launch) that workgroup slot `first` of `stride` takes:
// f(t0, ntok, adapter) for blocks first, first + stride, ... (wave-uniform).
// (The first block is requested with the count: slot `first` is always
// inside the list's storage.)
template <class F>
__device__ inline void for_each_block(const MaParams& p, int first, int stride, F&& f) {
  const cip c0 = (cip)(p.cbl + first);
  const int t00 = c0[0], t10 = c0[1], a0 = c0[2];
  const int n = *(cip)&p.hdr->n_colblocks;
  for (int cb = first; cb < n; cb += stride) {
    if (cb == first) {
      f(t00, t10 - t00, a0);
    } else {
      const cip c = (cip)(p.cbl + cb);
      const int t0 = c[0], t1 = c[1], a = c[2];
      f(t0, t1 - t0, a);
    }
  }
}

// The column-block list: one workgroup of 1024 threads.  Up to 4096 ids in
// one pass (4 consecutive ids per thread, all requested at once, two
// barriers); beyond, passes of 1024 ids (two barriers each, the ids of the
// next pass requested during the current one).
constexpr int kMaSegLocal = 4096;
template <bool LOCAL>
__global__ __launch_bounds__(1024) void k_ma_segment(MaParams p) {
  auto on_start = [&](int32_t idx, int32_t t, int32_t id) {
    p.cbl_w[idx].t0 = t;
    p.cbl_w[idx].adapter = id;
    p.cbl_w[idx].pad = 0;
  };
  auto on_end = [&](int32_t idx, int32_t t1) { p.cbl_w[idx].t1 = t1; };
  const int32_t n =
      LOCAL ? segment_runs_local<16, kMaSegLocal / 1024>(p.ids, p.T, p.num_adapters, kMaTok,
                                                         on_start, on_end)
            : segment_runs<16>(p.ids, p.T, p.num_adapters, kMaTok, on_start, on_end);
  if (threadIdx.x == 0) p.hdr_w->n_colblocks = n;
}

template <int ELL>
__global__ __launch_bounds__(64 * kMaW1) void k_ma_stage1(MaParams p) {
  // LDS: the x blocks of every wave [wave][j][16 rows][256 B] (chunk c of
  // row r at position c ^ (r % 16) of the row, so the operand reads hit
  // distinct banks), later the waves' partial tiles [wave][term][tile
  // h][lane]; gamma_i of the adapter [ELL][M]
  constexpr int kXBytes = kMaW1 * kMaBlk * 4096;
  static_assert(kMaW1 * ELL * 4 * 64 * 16 <= kXBytes, "LDS");
  __shared__ __attribute__((aligned(1024))) char sx[kXBytes];
  __shared__ __attribute__((aligned(16))) half_t gl[kMaGamHalfs];
  const uint32_t sx0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)sx;
  v4f* red = (v4f*)sx;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int M = p.M, R = p.R;
  const int mg = (p.nkb1 + 1) * kColBlock;  // gamma row length in LDS
  int npass = 0;

  for_each_block(p, blockIdx.x, gridDim.x, [&](int t0, int ntok, int a) {
    if (a < 0) return;  // out-of-range ids: nothing in stage 1
    const bool live = c16 < ntok;
    if (npass++ > 0) __syncthreads();  // the previous adapter's readers of LDS are done

    // A chunk's requests: this wave's blocks kb = kc + wv + 8j (blocks past
    // the last repeat it): the x rows of the block's tokens (256 B each;
    // entries past M repeat the last 8) straight to the wave's LDS area, 256
    // contiguous bytes per 16 lanes, then their sign words to registers.
    // The x requests need only t0, so they go out while the adapter's factor
    // pointers are still on their way.
    auto dma_chunk = [&](int kc) {
#pragma unroll
      for (int j = 0; j < kMaBlk; ++j) {
        int kb = kc + wv + kMaW1 * j;
        kb = kb < p.nkb1 ? kb : p.nkb1 - 1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // (rows past the block's tokens are not requested: their columns
          // are computed from whatever the area holds and never stored)
          const int r = 4 * u + (lane >> 4);
          const int c = (lane & 15) ^ r;
          int k = kb * kColBlock + 8 * c;
          k = k < M - 8 ? k : M - 8;
          if (r < ntok)
            dma16(p.x, (uint32_t)(t0 + r) * (uint32_t)p.ldx * 2u + (uint32_t)k * 2u,
                  sx0 + (uint32_t)((wv * kMaBlk + j) * 4096 + u * 1024));
        }
      }
    };
    dma_chunk(0);
    const char* B2 = table_ptr<const char*>(p.B2s, a);
    const half_t* beta = table_ptr<const half_t*>(p.betas, a);
    const half_t* gamma = table_ptr<const half_t*>(p.gammas, a);
    v4u w[kMaBlk];
    auto sign_chunk = [&](int kc) {
#pragma unroll
      for (int j = 0; j < kMaBlk; ++j) {
        int kb = kc + wv + kMaW1 * j;
        kb = kb < p.nkb1 ? kb : p.nkb1 - 1;
        w[j] = *(gv4up)(B2 + ((int64_t)kb << 10) + lane * 16);
      }
    };
    sign_chunk(0);
    // gamma_i staged as [ELL][mg] with zeros from M on (mg = whole blocks
    // plus one zero block, which the blocks past the last use), so entries
    // past M meet a zero operand
    const bool g16 = (((uintptr_t)gamma) & 15u) == 0;
    v8h gv[kMaStage];
#pragma unroll
    for (int u = 0; u < kMaStage; ++u) {
      const int e = (tid + 64 * kMaW1 * u) * 8;
      const int i = e / mg, k = e - i * mg;
      gv[u] = v8h{};
      if (e < ELL * mg && k < M) {  // whole chunks: M is a multiple of 8
        const half_t* gp = gamma + (int64_t)i * M + k;
        if (g16)
          gv[u] = *(const DBF_GLOBAL v8h*)gp;
        else
          for (int v = 0; v < 8; ++v) gv[u][v] = ((ghp)gp)[v];
      }
    }
    // beta_i of the rows this wave finishes (term wv / 4, tile wv % 4)
    float bsv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = wv >> 2, r = (wv & 3) * kRowTile + 4 * g + v;
      bsv[v] = (wv < 4 * ELL && r < R) ? (float)((ghp)beta)[(int64_t)i * R + r] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kMaStage; ++u) {
      const int e = (tid + 64 * kMaW1 * u) * 8;
      if (e < ELL * mg) *(v8h*)(gl + e) = gv[u];
    }
    __syncthreads();  // gamma visible
    v4f acc[ELL][4];
#pragma unroll
    for (int i = 0; i < ELL; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[i][h] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < p.nkb1; kc += kMaW1 * kMaBlk) {
      // (waits as asm with a memory clobber: the compiler neither moves LDS
      // reads across them nor knows the direct-to-LDS requests)
      if (kc > 0) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's reads of its area
        dma_chunk(kc);
        sign_chunk(kc);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // its requests (it alone reads its area)
#pragma unroll
      for (int j = 0; j < kMaBlk; ++j) {
        const int kb = kc + wv + kMaW1 * j;
        const char* xl = sx + (wv * kMaBlk + j) * 4096 + c16 * 256;
        const int gb = kb < p.nkb1 ? kb * kColBlock : mg - kColBlock;  // the zero block past the last
        auto step = [&](auto sc) {
          constexpr int s = decltype(sc)::value;
          const int kk = gb + 32 * s + 8 * g;
          const v8h xv = *(const v8h*)(xl + (((4 * s + g) ^ c16) << 4));
          v8h a4[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) a4[h] = expand_cvt<s>(w[j][h], p.nib_mask, p.nib_one);
#pragma unroll
          for (int i = 0; i < ELL; ++i) {
            const v8h b = xv * *(const v8h*)(gl + i * mg + kk);
#pragma unroll
            for (int h = 0; h < 4; ++h)
              acc[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a4[h], b, acc[i][h], 0, 0, 0);
          }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
      }
    }
    __syncthreads();  // every wave is done with its x area
#pragma unroll
    for (int i = 0; i < ELL; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) red[((wv * ELL + i) * 4 + h) * 64 + lane] = acc[i][h];
    __syncthreads();
    // wave w < 4 * ELL finishes (term w / 4, tile w % 4): the 8 partials in
    // wave order, times beta_i, rounded to fp16; rows R .. ldz-1 get zero
    if (wv < 4 * ELL) {
      const int i = wv >> 2, h = wv & 3;
      v4f u = red[(i * 4 + h) * 64 + lane];
#pragma unroll
      for (int w2 = 1; w2 < kMaW1; ++w2) u += red[((w2 * ELL + i) * 4 + h) * 64 + lane];
      const int r0 = h * kRowTile + 4 * g;
      if (live && r0 < p.ldz) {
        v4h zv;
#pragma unroll
        for (int v = 0; v < 4; ++v) zv[v] = (half_t)(u[v] * bsv[v]);
        *(v4h*)(p.z + ((int64_t)i * p.T + t0 + c16) * p.ldz + r0) = zv;
      }
    }
  });
}

// (At most 128 registers: four waves per SIMD, so the dependent requests of
// more workgroups overlap.)
template <int ELL>
__global__ __launch_bounds__(64 * kMaW2, 4) void k_ma_stage2(MaParams p) {
  constexpr int kRowsWg = kMaW2 * kMaQw * 64;  // output rows of a workgroup
  __shared__ __attribute__((aligned(16))) float sts[kMaW2][kMaTok * 64];  // each wave's tile
  __shared__ __attribute__((aligned(16))) half_t sal[ELL][kRowsWg];       // alpha_i of the rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int slot = blockIdx.x / p.nch2, ch = blockIdx.x - slot * p.nch2;
  const int N = p.N;
  const int q0 = ch * kMaW2 * kMaQw;  // the workgroup's first row quad
  const int r_lo = q0 * 64;
  float* st = sts[wv];
  int npass = 0;

  for_each_block(p, slot, p.n_cb_est, [&](int t0, int ntok, int a) {
    if (a < 0) {
      // tokens of out-of-range ids: y = 0 on this workgroup's rows
      if (!p.accumulate) {
        const int nr = N - r_lo < kRowsWg ? N - r_lo : kRowsWg;
        for (int e = tid; e < kMaTok * nr; e += 64 * kMaW2) {
          const int tt = e / nr, n = r_lo + e - tt * nr;
          if (tt < ntok) {
            const int64_t off = (int64_t)(t0 + tt) * p.ldy + n;
            if (p.y_f32)
              ((float*)p.y)[off] = 0.0f;
            else
              ((half_t*)p.y)[off] = (half_t)0.0f;
          }
        }
      }
      return;
    }
    const char* B1 = table_ptr<const char*>(p.B1s, a);
    const half_t* alpha = table_ptr<const half_t*>(p.alphas, a);
    const bool live = c16 < ntok;
    // requests: the z operands (term, step) of this lane's token, the sign
    // words of this wave's quads and the workgroup's alpha rows
    v8h bz[ELL][2];
#pragma unroll
    for (int i = 0; i < ELL; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int r = 32 * s + 8 * g;
        bz[i][s] = (live && r < p.ldz)
                       ? *(const DBF_GLOBAL v8h*)(p.z + ((int64_t)i * p.T + t0 + c16) * p.ldz + r)
                       : v8h{};
      }
    v4u w1[kMaQw];
#pragma unroll
    for (int j = 0; j < kMaQw; ++j) {
      const int q = q0 + wv + kMaW2 * j;
      w1[j] = q < p.nq2 ? *(gv4up)(B1 + ((int64_t)q << 10) + lane * 16) : v4u{0u, 0u, 0u, 0u};
    }
    // alpha: one 8-half chunk per thread and term pass (rows past N zero)
    const bool a16 = (((uintptr_t)alpha) & 15u) == 0 && N % 8 == 0;
    constexpr int kAch = ELL * kRowsWg / 8;
    constexpr int kAper = (kAch + 64 * kMaW2 - 1) / (64 * kMaW2);
    v8h av[kAper];
#pragma unroll
    for (int u = 0; u < kAper; ++u) {
      const int e = tid + 64 * kMaW2 * u;
      const int i = e / (kRowsWg / 8), n = r_lo + (e - i * (kRowsWg / 8)) * 8;
      av[u] = v8h{};
      if (e < kAch) {
        const half_t* ap = alpha + (int64_t)i * N + n;
        if (a16 && n + 8 <= N) {
          av[u] = *(const DBF_GLOBAL v8h*)ap;
        } else {
          for (int v = 0; v < 8; ++v)
            if (n + v < N) av[u][v] = ((ghp)ap)[v];
        }
      }
    }
    if (npass++ > 0) __syncthreads();  // the previous adapter's readers of sal are done
#pragma unroll
    for (int u = 0; u < kAper; ++u) {
      const int e = tid + 64 * kMaW2 * u;
      if (e < kAch) *(v8h*)(&sal[0][0] + e * 8) = av[u];
    }
    __syncthreads();
    const int nst = p.R > 32 ? 2 : 1;
#pragma unroll
    for (int j = 0; j < kMaQw; ++j) {
      const int q = q0 + wv + kMaW2 * j;
      if (q >= p.nq2) break;
      v4f ac[ELL][4];
#pragma unroll
      for (int i = 0; i < ELL; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) ac[i][h] = v4f{0.f, 0.f, 0.f, 0.f};
      {
        v8h a4[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) a4[h] = expand_cvt<0>(w1[j][h], p.nib_mask, p.nib_one);
#pragma unroll
        for (int i = 0; i < ELL; ++i)
#pragma unroll
          for (int h = 0; h < 4; ++h)
            ac[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a4[h], bz[i][0], ac[i][h], 0, 0, 0);
      }
      if (nst > 1) {
        v8h a4[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) a4[h] = expand_cvt<1>(w1[j][h], p.nib_mask, p.nib_one);
#pragma unroll
        for (int i = 0; i < ELL; ++i)
#pragma unroll
          for (int h = 0; h < 4; ++h)
            ac[i][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a4[h], bz[i][1], ac[i][h], 0, 0, 0);
      }
      // alpha-scaled sum over the terms (ascending), parked as [token][row]
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int rl = (q - q0) * 64 + h * kRowTile + 4 * g;  // row in the workgroup
        v4h al[ELL];
#pragma unroll
        for (int i = 0; i < ELL; ++i) al[i] = *(const v4h*)&sal[i][rl];
        v4f o;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float sum = ac[0][h][v] * (float)al[0][v];
#pragma unroll
          for (int i = 1; i < ELL; ++i) sum += ac[i][h][v] * (float)al[i][v];
          o[v] = sum;
        }
        *(v4f*)&st[c16 * 64 + h * kRowTile + 4 * g] = o;
      }
      __builtin_amdgcn_wave_barrier();
      // lane L: token L / 4, rows 16 (L % 4) .. +15 of the quad
      const int tt = lane >> 2, rr = (lane & 3) * 16;
      const int n0 = q * 64 + rr;
      if (tt < ntok && n0 < N) {
        float o[16];
#pragma unroll
        for (int v = 0; v < 16; v += 4) {
          const v4f u = *(const v4f*)&st[tt * 64 + rr + v];
          o[v] = u[0];
          o[v + 1] = u[1];
          o[v + 2] = u[2];
          o[v + 3] = u[3];
        }
        const int64_t yoff = (int64_t)(t0 + tt) * p.ldy + n0;
        const int nv = N - n0 < 16 ? N - n0 : 16;
        if (p.y_f32) {
          float* yp = (float*)p.y + yoff;
          if (p.accumulate)
            for (int v = 0; v < nv; ++v) o[v] += yp[v];
          if (nv == 16) {
            // y is written once and not read again here: non-temporal
            // (streamed) stores, measured faster on the 64-adapter batch
#pragma unroll
            for (int v = 0; v < 16; v += 4)
              __builtin_nontemporal_store(v4f{o[v], o[v + 1], o[v + 2], o[v + 3]}, (v4f*)(yp + v));
          } else {
            for (int v = 0; v < nv; ++v) yp[v] = o[v];
          }
        } else {
          half_t* yp = (half_t*)p.y + yoff;
          if (p.accumulate)
            for (int v = 0; v < nv; ++v) o[v] += (float)yp[v];
          if (nv == 16) {
            v8h h0, h1;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              h0[v] = (half_t)o[v];
              h1[v] = (half_t)o[v + 8];
            }
            __builtin_nontemporal_store(h0, (v8h*)yp);
            __builtin_nontemporal_store(h1, (v8h*)(yp + 8));
          } else {
            for (int v = 0; v < nv; ++v) yp[v] = (half_t)o[v];
          }
        }
      }
      // the wave's reads of st end before the next quad's writes
      __builtin_amdgcn_wave_barrier();
    }
  });
}

template <int ELL>
hipError_t launch_ell(const MaParams& p, int phases, hipStream_t s) {
  if (phases & 1) {
    if (p.T <= kMaSegLocal)
      hipLaunchKernelGGL(k_ma_segment<true>, dim3(1), dim3(1024), 0, s, p);
    else
      hipLaunchKernelGGL(k_ma_segment<false>, dim3(1), dim3(1024), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    hipLaunchKernelGGL((k_ma_stage1<ELL>), dim3((unsigned)p.n_cb_est), dim3(64 * kMaW1), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 4) {
    hipLaunchKernelGGL((k_ma_stage2<ELL>), dim3((unsigned)((int64_t)p.n_cb_est * p.nch2)),
                       dim3(64 * kMaW2), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

// Workgroups of stage 1: the column blocks of sorted ids (each adapter's
// run adds at most one partial block); more blocks (unsorted ids) are taken
// in turns.
int64_t ma_blocks_est(const ForwardArgs& a) {
  const int64_t n = cdiv(a.T, kMaTok) + (a.num_adapters < a.T ? a.num_adapters : a.T) + 1;
  return n < max_colblocks(a.T) ? n : max_colblocks(a.T);
}

// Whether the short-rank multi-adapter kernels take this call: R <= 64, at
// most two terms, M a multiple of 8 (x read in 16-byte chunks) with gamma_i
// of every term fitting its LDS area, x and y rows that take 16-byte loads
// and stores (x addressed with 32-bit byte offsets), and grids within 32
// bits.
bool ma_short_fits(const ForwardArgs& a) {
  const size_t esz = a.y_f32 ? 4 : 2;
  const int64_t nch2 = cdiv(cdiv(a.N, kRowTile * kQuad), kMaW2 * kMaQw);
  return a.multi && a.group <= 1 && a.R >= 1 && a.R <= 64 && a.ell >= 1 &&
         a.ell <= kMaMaxEll && a.M % 8 == 0 &&
         (int64_t)a.ell * (cdiv(a.M, kColBlock) + 1) * kColBlock <= kMaGamHalfs &&
         ma_blocks_est(a) * nch2 <= INT32_MAX &&
         a.T * a.ldx * 2 < ((int64_t)1 << 31) &&
         (((uintptr_t)a.x) & 15u) == 0 && a.ldx % 8 == 0 &&
         (((uintptr_t)a.y) & 15u) == 0 && (a.ldy * (int64_t)esz) % 16 == 0;
}

// The prep phase writes the column blocks (runs of at most 16 tokens of one
// adapter) into the workspace; stage 1 writes z [ell][T][ldz_of(R)] fp16
// into its z region; stage 2 reads both.
hipError_t launch_ma_short(const ForwardArgs& a, hipStream_t s) {
  const WsLayout L = ws_layout(a.N, a.R, a.M, a.ell, a.T);
  MaParams p{};
  p.x = a.x;
  p.ldx = a.ldx;
  p.ids = a.ids;
  p.num_adapters = a.num_adapters;
  p.B1s = a.B1s;
  p.B2s = a.B2s;
  p.alphas = a.alphas;
  p.betas = a.betas;
  p.gammas = a.gammas;
  p.z = (half_t*)((char*)a.ws + L.z);
  p.ldz = (int32_t)ldz_of(a.R);
  p.cbl_w = (ColBlock*)((char*)a.ws + L.cbl);
  p.hdr_w = (WsHeader*)a.ws;
  p.cbl = p.cbl_w;
  p.hdr = p.hdr_w;
  p.n_cb_est = (int32_t)ma_blocks_est(a);
  p.y = a.y;
  p.ldy = a.ldy;
  p.y_f32 = a.y_f32;
  p.accumulate = a.accumulate;
  p.N = (int32_t)a.N;
  p.R = (int32_t)a.R;
  p.M = (int32_t)a.M;
  p.T = (int32_t)a.T;
  p.ell = a.ell;
  p.nkb1 = (int32_t)cdiv(a.M, kColBlock);
  p.nq2 = (int32_t)cdiv(a.N, kRowTile * kQuad);
  p.nch2 = (int32_t)cdiv(p.nq2, kMaW2 * kMaQw);
  p.nib_mask = 0x88888888u;
  p.nib_one = 0x22222222u;
  return a.ell == 1 ? launch_ell<1>(p, a.phases, s) : launch_ell<2>(p, a.phases, s);
}

}  // namespace dbf
