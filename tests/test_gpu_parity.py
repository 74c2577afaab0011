"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: bit-exact on integer-valued inputs with unit scales (fp32 output equals
float32 of the exact value; fp16 output equals its nearest-even rounding);
max|y - y_ref| / max|y_ref| <= 2e-3 on fp16 inputs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3
PATHS = ["gemv", "mfma"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.manual_seed(0)


def H():
    import gpu_helpers
    return gpu_helpers


def ref(L, y_old=None):
    return oracle.forward(L.x, L.S1, L.S2, L.alpha, L.beta, L.gamma, y_old=y_old)


# ------------------------------------------------------------ packing ----

@pytest.mark.parametrize("rows,cols", [(1, 1), (37, 300), (16, 128), (64, 4096), (5, 33)])
def test_pack_layout_int8(rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    S = synth.make_signs(rng, rows, cols)
    packed = H().dbf.dbf_pack_signs(H().to_dev(S))
    torch.cuda.synchronize()
    got = packed.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, H().pack_ref(S))


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_pack_latent_sign(dtype):
    rng = np.random.default_rng(7)
    h = rng.standard_normal((40, 200)).astype(dtype)
    h[0, :5] = [0.0, -0.0, np.nan, -np.inf, np.inf]
    h[3, 7] = -np.finfo(dtype).tiny
    packed = H().dbf.dbf_pack_signs(H().to_dev(h))
    torch.cuda.synchronize()
    want = H().pack_ref(oracle.sign_of_latent(h))
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), want)


@pytest.mark.parametrize("rows,cols", [(64, 128), (65, 129), (200, 37), (1, 300), (513, 64)])
def test_transpose_signs(rows, cols):
    """Transposing packed signs equals packing the transposed matrix (byte
    for byte, padding included) and unpacks to S^T."""
    import double_binary_rank_amd as dbf
    S = synth.make_signs(np.random.default_rng(rows * 7 + cols), rows, cols)
    P = dbf.dbf_pack_signs(H().to_dev(S))
    PT = dbf.dbf_transpose_signs(P, rows, cols)
    want = dbf.dbf_pack_signs(H().to_dev(np.ascontiguousarray(S.T)))
    torch.cuda.synchronize()
    assert torch.equal(PT, want)
    assert np.array_equal(dbf.dbf_unpack_signs(PT, cols, rows).cpu().numpy(), S.T)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", [(72, 40, 136, 2, 9), (300, 130, 260, 1, 37)])
def test_transposed_forward(shape, path):
    """The transposed layer's forward maps g [T][N] to dW^T g per row
    (oracle.forward_transposed): fp16 inputs within the bar, integer inputs
    bit for bit, and <g, dW x> = <dW^T g, x> between the two GPU products."""
    N, R, M, ell, T = shape
    L = synth.make_layer(N, R, M, ell, T, seed=97)
    pl = H().upload(L)
    plt = pl.transposed()
    assert (plt.N, plt.R, plt.M) == (M, R, N)
    g = np.random.default_rng(99).standard_normal((T, N)).astype(np.float16)
    got = plt.forward(H().to_dev_rows(g), path=path, y=H().empty_rows(T, M, torch.float32),
                      y_dtype=torch.float32)
    torch.cuda.synchronize()
    want = oracle.forward_transposed(g, L.S1, L.S2, L.alpha, L.beta, L.gamma)
    got = got.cpu().numpy().astype(np.float64)
    assert oracle.max_norm_error(got, want) <= TOL
    y = H().run_layer(L, path=path, y_dtype=torch.float32, pl=pl)
    lhs = float(np.sum(g.astype(np.float64) * y))
    rhs = float(np.sum(got * L.x.astype(np.float64)))
    assert abs(lhs - rhs) <= 4 * TOL * (np.abs(g).sum() * np.abs(y).max() + 1.0)
    Li = synth.make_layer(N, R, M, ell, T, seed=100, alpha="ones", beta="ones", gamma="ones",
                          x_kind="int3")
    gi = np.random.default_rng(101).integers(-3, 4, (T, N)).astype(np.float16)
    pli = H().upload(Li).transposed()
    goti = pli.forward(H().to_dev_rows(gi), path=path, y=H().empty_rows(T, M, torch.float32),
                       y_dtype=torch.float32)
    torch.cuda.synchronize()
    wanti = oracle.forward_transposed(gi, Li.S1, Li.S2, Li.alpha, Li.beta, Li.gamma)
    assert np.array_equal(goti.cpu().numpy().astype(np.float64),
                          wanti.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("rows,cols", [(37, 300), (128, 64), (3, 1)])
def test_unpack_roundtrip(rows, cols):
    rng = np.random.default_rng(rows + cols)
    S = synth.make_signs(rng, rows, cols)
    d = H().dbf
    back = d.dbf_unpack_signs(d.dbf_pack_signs(H().to_dev(S)), rows, cols)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), S)


# -------------------------------------------------- single layer parity ----

@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.float16])
def test_tiny_integer_bitexact(path, y_dtype):
    L = synth.make_config_layer(1, 4, integer=True)
    y = H().run_layer(L, path=path, y_dtype=y_dtype)
    want = ref(L)
    if y_dtype == torch.float32:
        assert np.array_equal(y, want.astype(np.float32).astype(np.float64))
    else:
        assert np.array_equal(y, oracle.fp16_rne(want).astype(np.float64))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg,T", [(1, 4), (2, 1), (2, 8), (3, 1)])
def test_config_parity(cfg, T, path):
    L = synth.make_config_layer(cfg, T)
    err = oracle.max_norm_error(H().run_layer(L, path=path), ref(L))
    assert err <= TOL, err


@pytest.mark.parametrize("path", [None, "gemv", "mfma"])
def test_attn_T256_full(path):
    """4096 x 4096, R = 2048 at T = 256 (the prefill case the benchmark times)."""
    L = synth.make_config_layer(3, 256)
    err = oracle.max_norm_error(H().run_layer(L, path=path), ref(L))
    assert err <= TOL, err


@pytest.mark.parametrize("cfg", [4, 40])
@pytest.mark.parametrize("T", [1, 16, 256])
def test_mlp_sampled(cfg, T):
    """MLP up (14336 x 4096) and down (4096 x 14336), R = 6368: sampled
    tokens and outputs computed one by one by the oracle."""
    L = synth.make_config_layer(cfg, T)
    y = H().run_layer(L)
    rng = np.random.default_rng(T)
    toks = np.unique(rng.choice(T, size=min(T, 6), replace=False))
    cols = np.sort(rng.choice(L.N, size=384, replace=False))
    want = oracle.forward_rows(L.x[toks], L.S1, L.S2, L.alpha, L.beta, L.gamma, cols)
    err = oracle.max_norm_error(y[toks][:, cols], want)
    assert err <= TOL, err
    assert np.all(np.isfinite(y))


RAGGED = [(5, 7, 33, 1, 3), (300, 130, 260, 1, 37), (17, 129, 127, 2, 5), (64, 16, 8, 3, 70),
          (1, 1, 1, 1, 1), (33, 200, 520, 2, 130)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_integer_bitexact(shape, path):
    N, R, M, ell, T = shape
    L = synth.make_layer(N, R, M, ell, T, seed=sum(shape), alpha="ones", beta="ones", gamma="ones",
                         x_kind="int3")
    y = H().run_layer(L, path=path, y_dtype=torch.float32)
    assert np.array_equal(y, ref(L).astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_fp16(shape, path):
    N, R, M, ell, T = shape
    L = synth.make_layer(N, R, M, ell, T, seed=sum(shape) + 1)
    err = oracle.max_norm_error(H().run_layer(L, path=path), ref(L))
    assert err <= TOL, err


@pytest.mark.parametrize("path", PATHS)
def test_accumulate(path):
    L = synth.make_config_layer(1, 4, integer=True)
    rng = np.random.default_rng(3)
    base = rng.integers(-50, 50, size=(4, L.N)).astype(np.float16)
    y = H().run_layer(L, path=path, y_dtype=torch.float16, accumulate=True, y_init=base)
    assert np.array_equal(y, oracle.fp16_rne(ref(L, y_old=base)).astype(np.float64))


@pytest.mark.parametrize("path", PATHS)
def test_sign_flip_gauge_bitwise(path):
    """Negating column r of B1 together with row r of B2 leaves y bit-identical
    (fp16 data: every step is sign-symmetric)."""
    L = synth.make_config_layer(1, 4)
    y0 = H().run_layer(L, path=path)
    rng = np.random.default_rng(5)
    flip = rng.random(L.R) < 0.5
    L.S1[:, flip] *= -1
    L.S2[flip, :] *= -1
    assert np.array_equal(H().run_layer(L, path=path), y0)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", [(200, 100, 300, 2, 70), (136, 200, 264, 1, 40)])
def test_signed_scales(shape, path):
    """Negative entries in alpha, beta and gamma (the large-T path folds
    alpha into the expanded signs of short-rank stage 2 with a sign XOR),
    fp16 output, both paths; and the integer case bit for bit."""
    import dataclasses
    N, R, M, ell, T = shape
    rng = np.random.default_rng(95)
    L = synth.make_layer(N, R, M, ell, T, seed=94)

    def flip(a):
        return (a * np.where(rng.random(a.shape) < 0.5, -1, 1)).astype(np.float16)

    L = dataclasses.replace(L, alpha=flip(L.alpha), beta=flip(L.beta), gamma=flip(L.gamma))
    err = oracle.max_norm_error(H().run_layer(L, path=path), ref(L))
    assert err <= TOL, err
    Li = synth.make_layer(N, R, M, ell, T, seed=96, alpha="ones", beta="ones", gamma="ones",
                          x_kind="int3")
    sgn = lambda a: (a * np.where(rng.random(a.shape) < 0.5, -1, 1)).astype(np.float16)
    Li = dataclasses.replace(Li, alpha=sgn(Li.alpha), beta=sgn(Li.beta), gamma=sgn(Li.gamma))
    got = H().run_layer(Li, path=path, y_dtype=torch.float32)
    assert np.array_equal(got, ref(Li).astype(np.float32).astype(np.float64))


# Layer shapes (N, R, M, ell, T) at about 515 tokens whose stages take each
# compiled token-tile shape (NC tiles of 16 tokens, W row quads, KS reduction
# parts) under the launcher's cost model, every size ragged: stage 1 works
# over R rows and M reduction entries, stage 2 over N rows and R entries.
TILE_SHAPES = [
    (66, 1999, 136, 1, 513),   # stage 1 (4, 4, 2), stage 2 (2, 1, 8)
    (72, 2001, 264, 2, 517),   # stage 1 (4, 2, 4), stage 2 (2, 1, 8)
    (1999, 130, 136, 2, 515),  # stage 1 (4, 4, 2), stage 2 (4, 4, 2)
    (1999, 520, 136, 1, 515),  # stage 1 (4, 4, 2), stage 2 (4, 2, 4)
    (77, 265, 264, 2, 45),     # stage 1 (2, 2, 4), stage 2 (2, 2, 4)
    (72, 130, 2000, 1, 70),    # stage 1 (2, 1, 8), stage 2 (4, 4, 2)
]


@pytest.mark.parametrize("shape", TILE_SHAPES)
def test_tile_shapes_every_element(shape):
    """Every output of the token-tile stages in each compiled tile shape,
    with tails in rows, reduction and tokens: integer inputs with unit
    scales bit for bit (z = S2 x is held in fp16, exact while every |z| is
    at most 2048: asserted), fp16 inputs within the bar."""
    N, R, M, ell, T = shape
    Li = synth.make_layer(N, R, M, ell, T, seed=sum(shape), alpha="ones", beta="ones",
                          gamma="ones", x_kind="int3")
    assert np.abs(Li.S2.astype(np.float64) @ Li.x.T.astype(np.float64)).max() <= 2048
    got = H().run_layer(Li, path="mfma", y_dtype=torch.float32)
    assert np.array_equal(got, ref(Li).astype(np.float32).astype(np.float64))
    L = synth.make_layer(N, R, M, ell, T, seed=sum(shape) + 1)
    err = oracle.max_norm_error(H().run_layer(L, path="mfma"), ref(L))
    assert err <= TOL, err


@pytest.mark.parametrize("shape", [(136, 200, 520, 2, 70), (64, 130, 904, 1, 33),
                                   (40, 72, 264, 1, 5), (40, 8448, 520, 1, 70)])
def test_stage1_x_in_place_and_operand_tiles(shape):
    """Large-T stage 1 reads x in place, with gamma folded into the expanded
    signs, when M is a multiple of 8 and gamma is 16-byte aligned; a gamma
    one element off alignment takes the gamma*x operand tiles instead.  Both
    give the exact value on integers with signed unit gamma, and fp16
    results within the bar.  M = 520 and 904 end in a partial 128-block,
    taken by waves 4 and 7 of an 8-wave split reduction, and (R = 8448: more
    work items than compute units) by wave 0 of a 4-wave one; M = 264 runs
    unsplit."""
    import dataclasses
    N, R, M, ell, T = shape
    rng = np.random.default_rng(98)

    def misaligned(pl):
        buf = torch.empty(pl.gamma.numel() + 1, dtype=torch.float16, device="cuda")
        buf[1:] = pl.gamma.reshape(-1)
        return dataclasses.replace(pl, gamma=buf[1:].view(pl.gamma.shape))

    Li = synth.make_layer(N, R, M, ell, T, seed=99, alpha="ones", beta="ones", gamma="ones",
                          x_kind="int3")
    Li = dataclasses.replace(
        Li, gamma=(Li.gamma * np.where(rng.random(Li.gamma.shape) < 0.5, -1, 1)).astype(np.float16))
    want = ref(Li).astype(np.float32).astype(np.float64)
    pl = H().upload(Li)
    assert pl.gamma.data_ptr() % 16 == 0
    for q in (pl, misaligned(pl)):
        got = H().run_layer(Li, path="mfma", y_dtype=torch.float32, pl=q)
        assert np.array_equal(got, want)
    L = synth.make_layer(N, R, M, ell, T, seed=100)
    pl = H().upload(L)
    for q in (pl, misaligned(pl)):
        err = oracle.max_norm_error(H().run_layer(L, path="mfma", pl=q), ref(L))
        assert err <= TOL, err


def odd_scales(pl):
    """The layer with alpha, beta and gamma moved to views that start one
    half past a 16-byte boundary (2-byte aligned only)."""
    def shift(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        buf[1:] = t.reshape(-1)
        return buf[1:].view(t.shape)
    return dataclasses.replace(pl, alpha=shift(pl.alpha), beta=shift(pl.beta), gamma=shift(pl.gamma))


@pytest.mark.parametrize("shape", [(300, 130, 260, 1, 1), (4096, 2048, 4096, 1, 1),
                                   (96, 200, 8000, 1, 2), (72, 40, 136, 2, 1), (1, 1, 1, 1, 1),
                                   (64, 37, 96, 1, 1), (64, 38, 97, 1, 1), (80, 37, 98, 2, 1),
                                   (300, 2100, 1000, 1, 1), (64, 4200, 8200, 1, 1)])
def test_decode_stages_build_parts(shape):
    """With one adapter and ell * tokens <= 2 the small-T stages build their
    fp8 operand parts themselves, from gamma*x and from z, with no prep
    launch, and stage 1 splits its reduction into 1, 2, 4 or 8 parts whose
    partial z stage 2 adds: here 2 parts of 2 and 1 blocks (M = 260), 8 of
    4 (the attention layer), 8 parts of the 63-block M = 8000 with two
    tokens, 2 of one block each (ell = 2), 4 parts read by 2 blocks per
    stage-2 wave (R = 2100), and 2 parts of 33 and 32 blocks read by 4
    blocks per wave (R = 4200, M = 8200, a partial last block); M odd or
    gamma not 4-byte aligned takes the prep launch unsplit.  Odd R puts the
    last entry pair of stage 2 on the z row's padding.  Exact on integer
    inputs with unit scales, also with 2-byte aligned scale vectors, within
    the bar on fp16, and equal to the result of the adapter-table call,
    whose prep launches build the same parts, on integers."""
    N, R, M, ell, T = shape
    Li = synth.make_layer(N, R, M, ell, T, seed=101, alpha="ones", beta="ones", gamma="ones",
                          x_kind="int3")
    want = ref(Li).astype(np.float32).astype(np.float64)
    got = H().run_layer(Li, path="gemv", y_dtype=torch.float32)
    assert np.array_equal(got, want)
    got = H().run_layer(Li, path="gemv", y_dtype=torch.float32, pl=odd_scales(H().upload(Li)))
    assert np.array_equal(got, want)
    D = H().DeviceAdapters([Li])
    ids = H().to_dev(np.zeros(T, np.int32))
    y = D.forward(H().to_dev_rows(Li.x), ids, path="gemv", y=H().empty_rows(T, N, torch.float32))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want)
    L = synth.make_layer(N, R, M, ell, T, seed=102)
    err = oracle.max_norm_error(H().run_layer(L, path="gemv"), ref(L))
    assert err <= TOL, err
    err = oracle.max_norm_error(H().run_layer(L, path="gemv", pl=odd_scales(H().upload(L))), ref(L))
    assert err <= TOL, err


def test_paths_agree_on_integers():
    L = synth.make_layer(96, 200, 300, 2, 20, seed=9, alpha="ones", beta="ones", gamma="ones",
                         x_kind="int3")
    a = H().run_layer(L, path="gemv", y_dtype=torch.float32)
    b = H().run_layer(L, path="mfma", y_dtype=torch.float32)
    assert np.array_equal(a, b)


def test_determinism_and_stream():
    L = synth.make_config_layer(3, 1)
    pl = H().upload(L)
    x = H().to_dev(L.x)
    outs = []
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(20):
            outs.append(pl.forward(x).clone())
    s.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    err = oracle.max_norm_error(outs[0].float().cpu().numpy(), ref(L))
    assert err <= TOL


def test_guard_bands_untouched():
    L = synth.make_layer(40, 24, 72, 1, 7, seed=11)
    pl = H().upload(L)
    x = H().to_dev(L.x)
    canary = -12345.0
    big = torch.full((7 + 4, 64 + 16), canary, dtype=torch.float32, device="cuda")
    y = big[2:9, 8:48]  # ldy = 80, 40 columns written
    pl.forward(x, y=y, y_dtype=torch.float32)
    torch.cuda.synchronize()
    b = big.cpu().numpy()
    mask = np.ones_like(b, dtype=bool)
    mask[2:9, 8:48] = False
    assert np.all(b[mask] == canary)
    err = oracle.max_norm_error(b[2:9, 8:48], ref(L))
    assert err <= TOL


def test_T0_noop():
    L = synth.make_layer(16, 8, 32, 1, 0, seed=1)
    pl = H().upload(L)
    x = torch.empty((0, 32), dtype=torch.float16, device="cuda")
    y = pl.forward(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 16)


# ------------------------------------------------------- multi-adapter ----

def _multi_ref(B, ids, y_old=None):
    return oracle.forward_multi_adapter(B.x, ids, B.adapters, y_old=y_old)


@pytest.mark.parametrize("path", [None, "gemv", "mfma"])
def test_multi_adapter_config5(path):
    B = synth.make_multi_adapter()  # 64 adapters, 4096^2, R=64, ell=2, T=2048, Zipf ids
    D = H().DeviceAdapters(B.adapters)
    y = D.forward(H().to_dev(B.x), H().to_dev(B.ids), path=path)
    torch.cuda.synchronize()
    err = oracle.max_norm_error(y.float().cpu().numpy(), _multi_ref(B, B.ids))
    assert err <= TOL, err


@pytest.mark.parametrize("path", PATHS)
def test_multi_adapter_integer_unsorted_invalid(path):
    B = synth.make_multi_adapter(num_adapters=5, N=72, R=40, M=136, ell=2, T=77, seed=21,
                                 alpha="ones", beta="ones", gamma="ones", x_kind="int3",
                                 sort=False)
    ids = B.ids.copy()
    ids[[0, 9, 10, 40]] = [-1, 5, 1000, -7]
    D = H().DeviceAdapters(B.adapters)
    y = D.forward(H().to_dev(B.x), H().to_dev(ids), path=path, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64),
                          _multi_ref(B, ids).astype(np.float32).astype(np.float64))
    # accumulate: rows of invalid ids keep the base output
    base = np.random.default_rng(2).integers(-9, 9, size=(77, 72)).astype(np.float32)
    y2 = D.forward(H().to_dev(B.x), H().to_dev(ids), path=path, y=H().to_dev(base),
                   accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().astype(np.float64),
                          _multi_ref(B, ids, y_old=base).astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("path", PATHS)
def test_multi_adapter_many_adapters(path):
    """More adapters than the stage kernels keep pointer tables for in LDS
    (256): the factor pointers are then read from the device tables.  Exact
    on integer inputs, including ids out of range."""
    B = synth.make_multi_adapter(num_adapters=300, N=72, R=40, M=136, ell=2, T=700, seed=23,
                                 alpha="ones", beta="ones", gamma="ones", x_kind="int3",
                                 zipf_s=0.3)
    ids = B.ids.copy()
    ids[[3, 400]] = [-1, 300]
    assert len(np.unique(ids[(ids >= 0) & (ids < 300)])) > 256
    D = H().DeviceAdapters(B.adapters)
    y = D.forward(H().to_dev(B.x), H().to_dev(ids), path=path, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64),
                          _multi_ref(B, ids).astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("shape", [(70, 20, 4104, 1, 40), (200, 64, 264, 2, 77),
                                   (64, 33, 8, 2, 16), (96, 48, 16384, 2, 33)])
def test_multi_short_rank_kernel(shape):
    """The tile kernels of several short-rank adapters (R <= 64, at most two
    terms) on the large-T path: N not a multiple of 4 or of 64, one or two
    MFMA steps of rank, the reduction over M split over 1 to 8 workgroups
    per tile (the last one short, ending in a partial block), a partial last
    token tile, unsorted ids (many adapters per tile) with out-of-range
    ones; exact on integers (fp32 output, also accumulating onto a base) and
    within the bar on fp16 data."""
    N, R, M, ell, T = shape
    B = synth.make_multi_adapter(num_adapters=6, N=N, R=R, M=M, ell=ell, T=T, seed=61,
                                 alpha="ones", beta="ones", gamma="ones", x_kind="int3",
                                 sort=False)
    ids = B.ids.copy()
    ids[[1, T - 1]] = [-1, 6]
    D = H().DeviceAdapters(B.adapters)
    x, idd = H().to_dev_rows(B.x), H().to_dev(ids)
    y = D.forward(x, idd, path="mfma", y=H().empty_rows(T, N, torch.float32))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64),
                          _multi_ref(B, ids).astype(np.float32).astype(np.float64))
    base = np.random.default_rng(3).integers(-9, 9, size=(T, N)).astype(np.float32)
    y2 = D.forward(x, idd, path="mfma", y=H().to_dev_rows(base), accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().numpy().astype(np.float64),
                          _multi_ref(B, ids, y_old=base).astype(np.float32).astype(np.float64))
    # scales of both signs that differ row by row (alpha is folded into the
    # signs of stage 2 per row), still exact (|z| as with unit scales)
    Bs = synth.make_multi_adapter(num_adapters=6, N=N, R=R, M=M, ell=ell, T=T, seed=63,
                                  alpha="pm12", beta="pm1", gamma="pm1", x_kind="int3",
                                  sort=False)
    Ds = H().DeviceAdapters(Bs.adapters)
    ys = Ds.forward(H().to_dev_rows(Bs.x), H().to_dev(Bs.ids), path="mfma",
                    y=H().empty_rows(T, N, torch.float32))
    torch.cuda.synchronize()
    assert np.array_equal(ys.cpu().numpy().astype(np.float64),
                          _multi_ref(Bs, Bs.ids).astype(np.float32).astype(np.float64))
    Bf = synth.make_multi_adapter(num_adapters=6, N=N, R=R, M=M, ell=ell, T=T, seed=62)
    Df = H().DeviceAdapters(Bf.adapters)
    yf = Df.forward(H().to_dev_rows(Bf.x), H().to_dev(Bf.ids), path="mfma",
                    y=H().empty_rows(T, N, torch.float16))
    torch.cuda.synchronize()
    err = oracle.max_norm_error(yf.float().cpu().numpy(), _multi_ref(Bf, Bf.ids))
    assert err <= TOL, err


def test_multi_adapter_permutation_invariance():
    B = synth.make_multi_adapter(num_adapters=8, N=256, R=64, M=256, ell=2, T=300, seed=33)
    D = H().DeviceAdapters(B.adapters)
    x, ids = H().to_dev(B.x), H().to_dev(B.ids)
    y = D.forward(x, ids)
    perm = torch.as_tensor(np.random.default_rng(4).permutation(300)).cuda()
    yp = D.forward(x[perm].contiguous(), ids[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(yp, y[perm])


def test_multi_equals_single():
    """A batch routed entirely to adapter k equals dbf_forward of adapter k."""
    B = synth.make_multi_adapter(num_adapters=3, N=128, R=32, M=192, ell=1, T=40, seed=44)
    D = H().DeviceAdapters(B.adapters)
    x = H().to_dev(B.x)
    ids = torch.full((40,), 2, dtype=torch.int32, device="cuda")
    ym = D.forward(x, ids, path="gemv")
    ys = D.layers[2].forward(x, path="gemv")
    torch.cuda.synchronize()
    assert torch.equal(ym, ys)


@pytest.mark.parametrize("integer", [False, True])
def test_multi_adapter_stream_path(integer):
    """Many adapters with <= 5 tokens each: the decode path's streaming kernel
    (row quads spread over all waves, reduction chunked through LDS when the
    staged operands of a 36-block reduction do not fit at once)."""
    kind = dict(alpha="ones", beta="ones", gamma="ones", x_kind="int3") if integer else {}
    B = synth.make_multi_adapter(num_adapters=64, N=1024, R=1100, M=4608, ell=1, T=300, seed=55,
                                 **kind)
    ids = np.repeat(np.arange(64, dtype=np.int32), 5)[:300]
    D = H().DeviceAdapters(B.adapters)
    y = D.forward(H().to_dev(B.x), H().to_dev(ids), y_dtype=torch.float32)
    torch.cuda.synchronize()
    want = _multi_ref(B, ids)
    if integer:
        assert np.array_equal(y.cpu().numpy().astype(np.float64),
                              want.astype(np.float32).astype(np.float64))
    else:
        err = oracle.max_norm_error(y.cpu().numpy(), want)
        assert err <= TOL, err


def _fused_case(ell, integer, T=400, A=300, seed=61, max_run=7):
    kind = dict(alpha="ones", beta="ones", gamma="ones", x_kind="int3") if integer else {}
    B = synth.make_multi_adapter(num_adapters=A, N=200, R=136, M=264, ell=ell, T=T, seed=seed,
                                 **kind)
    rng = np.random.default_rng(seed + 1)
    runs = np.repeat(rng.integers(-2, A + 2, T), rng.integers(1, max_run + 1, T))[:T]
    return B, runs.astype(np.int32)


@pytest.mark.parametrize("ell,integer,T,max_run", [(1, False, 400, 7), (2, False, 400, 7),
                                                   (1, True, 400, 7), (2, True, 400, 7),
                                                   (1, True, 700, 2)])
def test_multi_adapter_fused_decode(ell, integer, T, max_run):
    """Many adapters (an estimate of at least 256 column blocks of <= 16/(3*ell)
    tokens): one fused launch segments the ids and runs both stages per
    column block.  Unsorted runs of 1..max_run tokens, out-of-range ids, 3
    stage-1 row quads for 12 waves (most waves stream only stage 2), ragged
    last quads, a 3-block reduction padded to the ring depth, and (T=700,
    runs of 1..2) more column blocks than workgroups.  Checked against the
    oracle, and against the same call split into phases (which takes the
    multi-launch path)."""
    B, ids = _fused_case(ell, integer, T=T, max_run=max_run)
    D = H().DeviceAdapters(B.adapters)
    x, idd = H().to_dev(B.x), H().to_dev(ids)
    T = len(ids)
    y = D.forward(x, idd, path="gemv", y_dtype=torch.float32)
    ws = torch.empty(dbf_ws(200, 136, 264, ell, T), dtype=torch.uint8, device="cuda")
    ys = torch.empty((T, 200), dtype=torch.float32, device="cuda")
    D.forward(x, idd, path="gemv", y=ys, ws=ws, phases=["prep", "stage1"])
    D.forward(x, idd, path="gemv", y=ys, ws=ws, phases="stage2")
    torch.cuda.synchronize()
    want = _multi_ref(B, ids)
    got, split = y.cpu().numpy().astype(np.float64), ys.cpu().numpy().astype(np.float64)
    if integer:
        assert np.array_equal(got, want.astype(np.float32).astype(np.float64))
        assert np.array_equal(split, got)
    else:
        err = oracle.max_norm_error(got, want)
        assert err <= TOL, err
        assert oracle.max_norm_error(split, want) <= TOL


@pytest.mark.parametrize("integer", [False, True])
def test_grouped_decode_full_size(integer):
    """The grouped decode at its real shape: 256 one-token adapters of the
    attention projection (4096, 2048, 4096) in one multi-adapter call, which
    takes the fused decode kernel with 32 and 16 reduction blocks per stage
    (four and two rounds of its 8-deep sign ring, and the stage-1 ring
    handing over to a long stage 2).  Eight distinct layers sit behind 32
    table entries each; the ids are a permutation of 0..255.  Every token and
    every output is compared with the oracle: bit for bit on integer inputs
    with unit scales, within the bar on fp16 data with log-normal scales."""
    kind = (dict(alpha="ones", beta="ones", gamma="ones", x_kind="int3") if integer else
            dict(alpha="lognormal", beta="lognormal", gamma="lognormal"))
    B = synth.make_multi_adapter(num_adapters=8, N=4096, R=2048, M=4096, ell=1, T=256,
                                 seed=3900 + int(integer), **kind)
    entries = [e % 8 for e in range(256)]
    ids = np.random.default_rng(3910).permutation(256).astype(np.int32)
    D = H().DeviceAdapters(B.adapters, entries=entries)
    y = D.forward(H().to_dev(B.x), H().to_dev(ids), y_dtype=torch.float32)
    torch.cuda.synchronize()
    want = _multi_ref(B, ids % 8)
    got = y.cpu().numpy().astype(np.float64)
    if integer:
        assert np.abs(want).max() < 2 ** 24
        assert np.array_equal(got, want.astype(np.float32).astype(np.float64))
    else:
        err = oracle.max_norm_error(got, want)
        assert err <= TOL, err
        # and row by row: no token is left to the maximum of the others
        for t in range(0, 256, 17):
            assert oracle.max_norm_error(got[t], want[t]) <= 4 * TOL


@pytest.mark.parametrize("T,N,y_f32", [(256, 8192, True), (250, 8000, False), (320, 8192, True)])
def test_wide_token_blocks_integer(T, N, y_f32):
    """Stage 2 with many row quads and tokens (ceil(T/64) * ceil(N/64) >= 512
    and a reduction of at least four 128-blocks): the large-T path's widest
    token blocks, bit for bit on integer inputs, with a partial last token
    block and a ragged last row quad in the second case."""
    L = synth.make_layer(N, 512, 256, 1, T, seed=3950 + T, alpha="ones", beta="ones",
                         gamma="ones", x_kind="int3")
    want = oracle.forward(L.x, L.S1, L.S2, L.alpha, L.beta, L.gamma)
    got = H().run_layer(L, path="mfma", y_dtype=torch.float32 if y_f32 else torch.float16)
    if y_f32:
        assert np.array_equal(got, want.astype(np.float32).astype(np.float64))
    else:
        assert np.array_equal(got, oracle.fp16_rne(want).astype(np.float64))


def test_multi_adapter_fused_accumulate_fp16():
    """Fused decode with ACCUMULATE into an fp16 output: rows of out-of-range
    ids keep their old values, the others add the product."""
    B, ids = _fused_case(1, True, seed=71)
    D = H().DeviceAdapters(B.adapters)
    T = len(ids)
    base = np.random.default_rng(72).integers(-4, 5, (T, 200)).astype(np.float16)
    y = H().to_dev(base)
    D.forward(H().to_dev(B.x), H().to_dev(ids), path="gemv", y=y, accumulate=True)
    torch.cuda.synchronize()
    want = _multi_ref(B, ids, y_old=base.astype(np.float64))
    assert np.array_equal(y.cpu().numpy().astype(np.float64),
                          want.astype(np.float16).astype(np.float64))


def _ref_blocks(ids, n_adapters, chunk):
    """Column blocks by definition: maximal runs of equal normalised id (ids
    outside [0, n_adapters) count as -1), each cut every `chunk` tokens."""
    norm = [int(i) if 0 <= i < n_adapters else -1 for i in ids]
    out, t, T = [], 0, len(norm)
    while t < T:
        u = t
        while u < T and norm[u] == norm[t]:
            u += 1
        out += [(s, min(s + chunk, u), norm[t]) for s in range(t, u, chunk)]
        t = u
    return out


@pytest.mark.parametrize("path,ell,chunk,R,T", [("gemv", 1, 5, 32, 1000), ("gemv", 2, 2, 32, 1000),
                                                 ("mfma", 2, 32, 80, 1000),
                                                 ("mfma", 2, 16, 32, 1000),
                                                 ("mfma", 2, 16, 32, 4096),
                                                 ("mfma", 1, 16, 64, 5000)])
def test_segmentation_blocks(path, ell, chunk, R, T):
    """The column-block list the prep launch writes into the workspace (its
    header and list sit at the library's internal offsets 0 and 256) equals
    the list by definition: runs of 1..70 tokens over several passes of ids
    (or, for ranks up to 64 on the large-T path and up to 4096 ids, one
    pass of 4 ids per thread: the largest such T and one past it), equal
    neighbouring runs that merge, and out-of-range ids."""
    rng = np.random.default_rng(91)
    A, parts = 7, []
    while sum(len(p) for p in parts) < T:
        parts.append(np.full(int(rng.integers(1, 71)), int(rng.integers(-3, A + 3)), np.int32))
    ids = np.concatenate(parts)[:T]
    ids[300:340] = 4  # a run across the first pass boundary
    ids[511:513] = -1
    # (on the large-T path, ranks up to 64 cut runs every 16 tokens)
    B = synth.make_multi_adapter(num_adapters=A, N=64, R=R, M=128, ell=ell, T=len(ids), seed=92)
    D = H().DeviceAdapters(B.adapters)
    T = len(ids)
    ws = torch.full((dbf_ws(64, R, 128, ell, T),), 0xAB, dtype=torch.uint8, device="cuda")
    D.forward(H().to_dev(B.x), H().to_dev(ids), path=path, ws=ws, phases="prep")
    torch.cuda.synchronize()
    want = _ref_blocks(ids, A, chunk)
    n = int(ws[:4].view(torch.int32).item())
    assert n == len(want)
    got = ws[256:256 + 16 * n].view(torch.int32).reshape(n, 4).cpu().numpy()
    assert [tuple(int(v) for v in r[:3]) for r in got] == want
    assert not got[:, 3].any()


# ------------------------------------------------------- split phases --
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("shape", [(300, 130, 260, 1, 37), (64, 16, 8, 3, 70), (96, 200, 8000, 1, 2),
                                   (300, 130, 260, 2, 1), (4096, 2048, 4096, 1, 1)])
def test_stage_split_equals_whole(shape, path):
    """The three phases run one at a time on one workspace give the whole
    call's result bit for bit, and the phases before stage 2 leave y
    untouched (at decode sizes the whole call is one cooperative launch of
    both stages, the phases two launches)."""
    N, R, M, ell, T = shape
    L = synth.make_layer(N, R, M, ell, T, seed=81)
    pl = H().upload(L)
    x = H().to_dev_rows(L.x)
    y_whole = pl.forward(x, path=path, y=H().empty_rows(T, N, torch.float16))
    ws = torch.empty(dbf_ws(N, R, M, ell, T), dtype=torch.uint8, device="cuda")
    y = H().empty_rows(T, N, torch.float16)
    y.fill_(7.0)
    pl.forward(x, path=path, y=y, ws=ws, phases="prep")
    pl.forward(x, path=path, y=y, ws=ws, phases="stage1")
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    pl.forward(x, path=path, y=y, ws=ws, phases=["stage2"])
    torch.cuda.synchronize()
    assert torch.equal(y, y_whole)


@pytest.mark.parametrize("path", PATHS)
def test_stage_split_multi_adapter(path):
    B = synth.make_multi_adapter(num_adapters=6, N=96, R=48, M=160, ell=2, T=90, seed=83)
    D = H().DeviceAdapters(B.adapters)
    x, ids = H().to_dev(B.x), H().to_dev(B.ids)
    y_whole = D.forward(x, ids, path=path, y=H().empty_rows(90, 96, torch.float16))
    ws = torch.empty(dbf_ws(96, 48, 160, 2, 90), dtype=torch.uint8, device="cuda")
    y = H().empty_rows(90, 96, torch.float16)
    D.forward(x, ids, path=path, y=y, ws=ws, phases=["prep", "stage1"])
    D.forward(x, ids, path=path, y=y, ws=ws, phases="stage2")
    torch.cuda.synchronize()
    assert torch.equal(y, y_whole)


def dbf_ws(N, R, M, ell, T):
    import double_binary_rank_amd as dbf
    return dbf.dbf_workspace_bytes(N, R, M, ell, T)


# ------------------------------------------------------------ backward --
def _bwd_ref(L, G, **kw):
    return oracle.backward(L.x, G, L.S1, L.S2, L.alpha, L.beta, L.gamma, **kw)


def _run_bwd(L, G, dx_dtype=torch.float32, H1=None, H2=None, tau=None):
    pl = H().upload(L)
    x = H().to_dev_rows(L.x)
    g = H().to_dev_rows(np.asarray(G, np.float16))
    kw = {}
    if H1 is not None:
        kw = dict(H1=torch.as_tensor(H1, dtype=torch.float32).cuda(),
                  H2=torch.as_tensor(H2, dtype=torch.float32).cuda(), tau=tau)
    out = pl.backward(x, g, dx_dtype=dx_dtype, sign_grads=True, **kw)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}


# every reduction's worst case stays below 2^24 and every fp16 operand value
# below 2048 (x, g in -3..3, unit scales), so the exact result is an fp32 value
BWD_INT_SHAPES = [(40, 24, 72, 1, 5), (300, 130, 260, 2, 9), (17, 129, 127, 2, 5),
                  (64, 16, 8, 3, 70), (1, 1, 1, 1, 1), (96, 200, 136, 1, 40), (24, 16, 40, 2, 200),
                  (72, 40, 72, 2, 37), (40, 24, 40, 1, 130)]  # M = N: sign products in pairs


@pytest.mark.parametrize("shape", BWD_INT_SHAPES)
def test_backward_integer_bitexact(shape):
    """Integer x and g with unit scales: dx, dalpha, dbeta, dgamma, dS1 and
    dS2 equal the oracle's exact values bit for bit (ragged sizes, several
    terms, token counts across the 128-token blocks of the sign gradients)."""
    N, R, M, ell, T = shape
    L = synth.make_layer(N, R, M, ell, T, seed=200 + sum(shape), alpha="ones", beta="ones",
                         gamma="ones", x_kind="int3")
    G = np.random.default_rng(201).integers(-3, 4, size=(T, N)).astype(np.float64)
    want = _bwd_ref(L, G)
    got = _run_bwd(L, G)
    for k in ("dx", "dalpha", "dbeta", "dgamma", "dS1", "dS2"):
        assert np.array_equal(got[k], want[k].astype(np.float32).astype(np.float64)), k


BWD_FP_SHAPES = [(300, 130, 260, 2, 37), (64, 16, 8, 3, 70), (96, 200, 136, 1, 300),
                 (520, 256, 384, 1, 129), (264, 130, 264, 2, 45)]


@pytest.mark.parametrize("shape", BWD_FP_SHAPES)
def test_backward_fp16(shape):
    """fp16 data: every gradient, including the straight-through latent
    gradients (tau = 0.5), within max|d - d_ref| / max|d_ref| <= 2e-3; dx as
    fp16 and as fp32."""
    N, R, M, ell, T = shape
    L = synth.make_layer(N, R, M, ell, T, seed=210 + sum(shape))
    rng = np.random.default_rng(211)
    G = oracle.fp16_rne(rng.standard_normal((T, N)))
    H1, H2 = rng.standard_normal((N, R)), rng.standard_normal((R, M))
    H1f, H2f = H1.astype(np.float32), H2.astype(np.float32)
    want = _bwd_ref(L, G, H1=H1f, H2=H2f, tau=0.5)
    for dx_dtype in (torch.float32, torch.float16):
        got = _run_bwd(L, G, dx_dtype=dx_dtype, H1=H1f, H2=H2f, tau=0.5)
        for k in ("dx", "dalpha", "dbeta", "dgamma", "dS1", "dS2", "dH1", "dH2"):
            err = oracle.max_norm_error(got[k], want[k])
            assert err <= TOL, (k, err)


@pytest.mark.parametrize("sign_grads,which", [(True, "H1"), (False, "H2"), (True, None)])
def test_backward_partial_sign_grads(sign_grads, which):
    """Sign gradients with only some outputs requested: dS1 and dS2 with the
    straight-through dH1 alone (the two dense products then take different
    epilogues), dH2 alone without dS, and dS alone; each requested output
    within the bar, the others absent."""
    N, R, M, ell, T = 96, 200, 136, 2, 40
    L = synth.make_layer(N, R, M, ell, T, seed=215)
    rng = np.random.default_rng(216)
    G = oracle.fp16_rne(rng.standard_normal((T, N)))
    H1 = rng.standard_normal((N, R)).astype(np.float32)
    H2 = rng.standard_normal((R, M)).astype(np.float32)
    want = _bwd_ref(L, G, H1=H1, H2=H2, tau=0.5)
    pl = H().upload(L)
    kw = {}
    if which == "H1":
        kw = dict(H1=torch.as_tensor(H1).cuda(), tau=0.5)
    elif which == "H2":
        kw = dict(H2=torch.as_tensor(H2).cuda(), tau=0.5)
    out = pl.backward(H().to_dev_rows(L.x), H().to_dev_rows(np.asarray(G, np.float16)),
                      dx_dtype=torch.float32, sign_grads=sign_grads, **kw)
    torch.cuda.synchronize()
    expect = {"dx", "dalpha", "dbeta", "dgamma"}
    expect |= {"dS1", "dS2"} if sign_grads else set()
    expect |= {"d" + which} if which else set()
    assert set(out) == expect
    for k in sorted(expect):
        err = oracle.max_norm_error(out[k].float().cpu().numpy().astype(np.float64), want[k])
        assert err <= TOL, (k, err)


def test_backward_attention_layer():
    """The attention projection (4096 x 4096, R = 2048, log-normal scales) at
    T = 64 tokens: every gradient within the bar."""
    L = synth.make_config_layer(3, 64)
    G = oracle.fp16_rne(np.random.default_rng(212).standard_normal((64, L.N)))
    want = _bwd_ref(L, G)
    got = _run_bwd(L, G)
    for k in ("dx", "dalpha", "dbeta", "dgamma", "dS1", "dS2"):
        err = oracle.max_norm_error(got[k], want[k])
        assert err <= TOL, (k, err)


# ------------------------------------------------------- factorisation --
def _scaled_sign(rng, n, k):
    u, v = np.exp(rng.normal(0, 0.3, n)), np.exp(rng.normal(0, 0.3, k))
    return u[:, None] * np.where(rng.random((n, k)) < 0.5, -1, 1) * v[None, :]


def _dense_of(f):
    """float64 dense update of a factorisation result (its fp16 scales)."""
    a = f["alpha"].float().cpu().numpy().astype(np.float64)[0]
    b = f["beta"].float().cpu().numpy().astype(np.float64)[0]
    g = f["gamma"].float().cpu().numpy().astype(np.float64)[0]
    S1 = f["S1"].cpu().numpy().astype(np.float64)
    S2 = f["S2"].cpu().numpy().astype(np.float64)
    return (a[:, None] * S1 * b[None, :]) @ (S2 * g[None, :])


def test_factorize_exact_start_is_a_fixed_point():
    """Started at an exact factorisation W = X* Y*, the GPU iteration keeps
    the sign matrices and reconstructs W (fp32 arithmetic, fp16 scales)."""
    rng = np.random.default_rng(300)
    N, M, k = 96, 80, 16
    X, Y = _scaled_sign(rng, N, k), _scaled_sign(rng, k, M)
    W = X @ Y
    dev = lambda a: torch.as_tensor(a, dtype=torch.float32).cuda()  # noqa: E731
    f = dbf_mod().dbf_factorize(dev(W), k, start=(dev(X), dev(Y)), outer=2, admm_iters=4)
    torch.cuda.synchronize()
    assert np.array_equal(f["S1"].cpu().numpy(), np.where(X < 0, -1, 1))
    assert np.array_equal(f["S2"].cpu().numpy(), np.where(Y < 0, -1, 1))
    assert float(f["rel_err"]) < 1e-5
    assert oracle.max_norm_error(_dense_of(f), W) < 2e-3  # fp16 scales


@pytest.mark.parametrize("shape", [(64, 48, 12), (200, 136, 40)])
def test_factorize_one_step_matches_oracle(shape):
    """From the same sketch, one ADMM iteration per side: the GPU's factors
    agree with the oracle's (fp32 vs fp64, power iteration vs SVD): at least
    99.5% of the signs, the dense updates within 1e-2 of max, and the same
    error to 1e-3."""
    N, M, k = shape
    rng = np.random.default_rng(301 + N)
    W = rng.standard_normal((N, M))
    om = rng.standard_normal((k, N))
    want = oracle.factorize(W, k, om, 1, 1)
    dev = lambda a: torch.as_tensor(a, dtype=torch.float32).cuda()  # noqa: E731
    f = dbf_mod().dbf_factorize(dev(W), k, dev(om), outer=1, admm_iters=1, power_iters=30)
    torch.cuda.synchronize()
    agree1 = (f["S1"].cpu().numpy() == want["S1"]).mean()
    agree2 = (f["S2"].cpu().numpy() == want["S2"]).mean()
    assert agree1 >= 0.995 and agree2 >= 0.995, (agree1, agree2)
    dw_want = (want["alpha"][:, None] * want["S1"] * want["beta"][None, :]) @ (
        want["S2"] * want["gamma"][None, :])
    assert oracle.max_norm_error(_dense_of(f), dw_want) < 1e-2
    assert abs(float(f["rel_err"]) - want["rel_err"]) < 1e-3


@pytest.mark.parametrize("shape", [(64, 48, 12), (128, 96, 24)])
def test_factorize_follows_the_dual(shape, monkeypatch):
    """Four ADMM iterations per side, so the dual variable carries over
    between iterations: the GPU's factors track the oracle's (signs, dense
    update, error) and sit far closer to it than to a plain alternating
    projection without the dual, which moves the dense update by 0.6-0.8
    of its maximum on these shapes."""
    N, M, k = shape
    rng = np.random.default_rng(301 + N)
    W = rng.standard_normal((N, M))
    om = rng.standard_normal((k, N))
    want = oracle.factorize(W, k, om, 1, 4)
    import oracle.dbf_oracle as od
    one = od.admm_scaled_sign

    def no_dual(W_, F, side, Z, iters, rho0):
        for _ in range(iters):
            Z = one(W_, F, side, Z, 1, rho0)
        return Z
    monkeypatch.setattr(od, "admm_scaled_sign", no_dual)
    plain = oracle.factorize(W, k, om, 1, 4)
    monkeypatch.setattr(od, "admm_scaled_sign", one)
    dev = lambda a: torch.as_tensor(a, dtype=torch.float32).cuda()  # noqa: E731
    f = dbf_mod().dbf_factorize(dev(W), k, dev(om), outer=1, admm_iters=4, power_iters=30)
    torch.cuda.synchronize()
    dense = lambda d: (d["alpha"][:, None] * d["S1"] * d["beta"][None, :]) @ (  # noqa: E731
        d["S2"] * d["gamma"][None, :])
    got = _dense_of(f)
    d_true = oracle.max_norm_error(got, dense(want))
    d_plain = oracle.max_norm_error(got, dense(plain))
    agree1 = (f["S1"].cpu().numpy() == want["S1"]).mean()
    agree2 = (f["S2"].cpu().numpy() == want["S2"]).mean()
    assert agree1 >= 0.98 and agree2 >= 0.98, (agree1, agree2)
    assert d_true < 0.1 and d_true < d_plain / 4, (d_true, d_plain)
    assert abs(float(f["rel_err"]) - want["rel_err"]) < 2e-3


def test_factorize_converges_like_oracle():
    """Several alternations: the GPU's error lands within 0.01 of the
    oracle's, it falls from the one-step error, and the reported error is
    that of the returned factors."""
    N, M, k = 128, 96, 24
    rng = np.random.default_rng(310)
    W = rng.standard_normal((N, M))
    om = rng.standard_normal((k, N))
    want = oracle.factorize(W, k, om, 4, 8)
    dev = lambda a: torch.as_tensor(a, dtype=torch.float32).cuda()  # noqa: E731
    f = dbf_mod().dbf_factorize(dev(W), k, dev(om), outer=4, admm_iters=8, power_iters=16)
    f1 = dbf_mod().dbf_factorize(dev(W), k, dev(om), outer=1, admm_iters=1, power_iters=16)
    torch.cuda.synchronize()
    err = float(f["rel_err"])
    assert abs(err - want["rel_err"]) < 0.01, (err, want["rel_err"])
    assert err < float(f1["rel_err"])
    dense_err = np.linalg.norm(W - _dense_of(f)) / np.linalg.norm(W)
    assert abs(dense_err - err) < 2e-3  # the fp16 rounding of the scales


def test_factorised_layer_runs_forward():
    """The factors, packed, are a layer: dbf_forward on them matches the
    oracle forward of the same factors."""
    N, M, k, T = 256, 192, 64, 9
    rng = np.random.default_rng(320)
    W = rng.standard_normal((N, M))
    om = rng.standard_normal((k, N))
    dev = lambda a: torch.as_tensor(a, dtype=torch.float32).cuda()  # noqa: E731
    f = dbf_mod().dbf_factorize(dev(W), k, dev(om), outer=2, admm_iters=4)
    pl = dbf_mod().PackedLayer.from_factorization(f)
    x = oracle.fp16_rne(rng.standard_normal((T, M)))
    y = pl.forward(H().to_dev_rows(x))
    torch.cuda.synchronize()
    ref_y = oracle.forward(x, f["S1"].cpu().numpy(), f["S2"].cpu().numpy(),
                           f["alpha"].float().cpu().numpy(), f["beta"].float().cpu().numpy(),
                           f["gamma"].float().cpu().numpy())
    assert oracle.max_norm_error(y.float().cpu().numpy(), ref_y) <= TOL


def dbf_mod():
    import double_binary_rank_amd as dbf
    return dbf


# ---------------------------------------------------- grouped layers --
GROUP_CASES = [
    (300, 130, 264, 1, 1, 3),   # decode, stages build their parts: one launch each
    (256, 512, 1024, 2, 1, 2),  # two terms, one token
    (200, 136, 520, 1, 2, 3),   # two tokens
    (136, 300, 520, 1, 70, 3),  # large T, x read in place, a partial last block
    (64, 390, 904, 1, 33, 8),   # eight layers
    (40, 300, 260, 1, 37, 2),   # M not a multiple of 8: layers one by one
    (96, 64, 128, 2, 20, 2),    # short-rank stage 2: layers one by one
    (72, 400, 8000, 1, 300, 2),  # a long reduction: prep launch, layers one by one
]


@pytest.mark.parametrize("case", GROUP_CASES)
def test_grouped_equals_single_calls(case):
    """Several layers on one x in one call: each layer's output is bit for bit
    that of dbf_forward on it, and within the bar of the oracle."""
    N, R, M, ell, T, J = case
    Ls = [synth.make_layer(N, R, M, ell, T, seed=400 + 10 * j + sum(case)) for j in range(J)]
    x = H().to_dev_rows(Ls[0].x)
    pls = [H().upload(L) for L in Ls]
    y = dbf_mod().dbf_forward_grouped(x, pls)
    singles = [p.forward(x) for p in pls]
    torch.cuda.synchronize()
    for j in range(J):
        assert torch.equal(y[j], singles[j]), j
        want = oracle.forward(Ls[0].x, Ls[j].S1, Ls[j].S2, Ls[j].alpha, Ls[j].beta, Ls[j].gamma)
        assert oracle.max_norm_error(y[j].float().cpu().numpy(), want) <= TOL


@pytest.mark.parametrize("T", [1, 64])
def test_grouped_accumulate_integer(T):
    """The fused add onto base outputs: integer data with unit scales, fp16
    output, y_j = fp16(base_j + y_j) exactly, in a strided output buffer."""
    N, R, M, J = 96, 300, 256, 3
    Ls = [synth.make_layer(N, R, M, 1, T, seed=450 + j, alpha="ones", beta="ones", gamma="ones",
                           x_kind="int3") for j in range(J)]
    x = H().to_dev_rows(Ls[0].x)
    pls = [H().upload(L) for L in Ls]
    rng = np.random.default_rng(451)
    base = rng.integers(-50, 50, size=(J, T, N)).astype(np.float16)
    buf = torch.zeros((J, T + 3, 104), dtype=torch.float16, device="cuda")
    y = buf[:, :T, :N]
    y.copy_(torch.as_tensor(base).cuda())
    dbf_mod().dbf_forward_grouped(x, pls, y=y, accumulate=True)
    torch.cuda.synchronize()
    for j in range(J):
        want = oracle.fp16_rne(oracle.forward(Ls[0].x, Ls[j].S1, Ls[j].S2, Ls[j].alpha,
                                              Ls[j].beta, Ls[j].gamma, y_old=base[j]))
        assert np.array_equal(y[j].float().cpu().numpy().astype(np.float64), want), j
    assert not bool(buf[:, T:, :].any()) and not bool(buf[:, :T, N:].any())


# -------------------------------- non-uniform ranks, decoder-layer stack --
def test_select_channels_equals_oracle():
    """A layer restricted to some middle channels equals the oracle on the
    same columns of S1, rows of S2 and entries of beta."""
    L = synth.make_layer(200, 130, 264, 1, 9, seed=500)
    pl = H().upload(L)
    keep = np.sort(np.random.default_rng(501).choice(130, 70, replace=False))
    sub = pl.select_channels(keep)
    y = sub.forward(H().to_dev_rows(L.x))
    torch.cuda.synchronize()
    want = oracle.forward(L.x, L.S1[:, keep], L.S2[keep], L.alpha, L.beta[:, keep], L.gamma)
    assert sub.R == 70
    assert oracle.max_norm_error(y.float().cpu().numpy(), want) <= TOL


DEC_SMALL = [(64, 64), (64, 64), (64, 64), (64, 64), (160, 64), (160, 64), (64, 160)]


@pytest.mark.parametrize("T", [1, 40])
def test_pruned_decoder_stack_chain(T):
    """Two synthetic decoder layers (q, k, v, o, gate, up, down; o and down
    added onto the residual with DBF_ACCUMULATE), built at 2 bits per weight
    and pruned non-uniformly to 1.5: the GPU chain equals an oracle chain that
    rounds to fp16 where the GPU does, within the bar, and the plan fits the
    budget with unequal widths."""
    import double_binary_rank_amd as dbf
    layers, host = [], []
    for li in range(2):
        for j, (N, M) in enumerate(DEC_SMALL):
            R = dbf.rank_for_bits(N, M, 2.0)
            # alpha = 1: each projection has a gain near 1, so the DBF
            # branches move h as much as the residual does
            L = synth.make_layer(N, R, M, 1, 0, seed=510 + 10 * li + j, alpha="ones",
                                 x_kind="none")
            host.append(L)
            layers.append(H().upload(L))
    shapes = [(p.N, p.R, p.M) for p in layers]
    budget = 1.5 * sum(N * M for (N, _, M) in shapes)
    keep = dbf.plan_channels(shapes, [p.channel_importance() for p in layers], budget)
    assert sum(dbf.layer_bits(N, len(k), M) for (N, _, M), k in zip(shapes, keep)) <= budget
    assert len({len(k) for k in keep}) > 1  # non-uniform
    pruned = [p.select_channels(k) for p, k in zip(layers, keep)]
    x = oracle.fp16_rne(np.random.default_rng(520).standard_normal((T, 64)))
    h = H().to_dev_rows(x)
    hr = x.copy()

    def ref(j, inp):
        L, k = host[j], keep[j]
        return oracle.forward(inp, L.S1[:, k], L.S2[k], L.alpha, L.beta[:, k], L.gamma)

    for li in range(2):
        b = 7 * li
        q = pruned[b].forward(h)
        pruned[b + 1].forward(h)
        pruned[b + 2].forward(h)
        qr = oracle.fp16_rne(ref(b, hr))
        h = h.clone()
        pruned[b + 3].forward(q, y=h, accumulate=True)
        hr = oracle.fp16_rne(hr + ref(b + 3, qr))
        pruned[b + 4].forward(h)
        u = pruned[b + 5].forward(h)
        ur = oracle.fp16_rne(ref(b + 5, hr))
        pruned[b + 6].forward(u, y=h, accumulate=True)
        hr = oracle.fp16_rne(hr + ref(b + 6, ur))
    torch.cuda.synchronize()
    assert oracle.max_norm_error(h.float().cpu().numpy(), hr) <= TOL
    assert oracle.max_norm_error(x, hr) > 0.5  # the layers changed h
