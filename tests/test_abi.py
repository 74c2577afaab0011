"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments synchronously (before any launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

from double_binary_rank_amd import _lib  # noqa: E402

L = _lib.lib


def _header_functions():
    with open(os.path.join(ROOT, "include", "dbf.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(dbf_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = _header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings():
    assert L.dbf_abi_version() == _lib.ABI_VERSION
    for s in (0, -1, -2, -3, -4):
        assert _lib.status_string(s).startswith("DBF_")
    assert _lib.status_string(-99) == "unknown dbf_status"


@pytest.mark.parametrize("rows,cols", [(1, 1), (64, 128), (65, 129), (4096, 2048), (14336, 6368)])
def test_packed_bytes_closed_form(rows, cols):
    want = -(-rows // 64) * -(-cols // 128) * 1024
    assert _lib.packed_bytes(rows, cols) == want
    assert want * 8 >= rows * cols  # at least one bit per sign
    # padding is less than one 64-row x 128-col unit in each direction
    assert want * 8 < (rows + 64) * (cols + 128)


def test_packed_bytes_errors():
    out = ctypes.c_size_t(0)
    assert L.dbf_packed_bytes(0, 5, ctypes.byref(out)) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_packed_bytes(5, -1, ctypes.byref(out)) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_packed_bytes(5, 5, None) == _lib.DBF_ERR_INVALID_ARG


def test_workspace_bytes():
    assert _lib.workspace_bytes(4096, 2048, 4096, 1, 0) > 0
    a = _lib.workspace_bytes(4096, 2048, 4096, 1, 256)
    assert a >= 256 * 2048 * 4  # holds the fp32 R-vectors of every token
    assert _lib.workspace_bytes(4096, 2048, 4096, 2, 256) > a
    out = ctypes.c_size_t(0)
    assert L.dbf_workspace_bytes(1, 1, 1, 0, 1, ctypes.byref(out)) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_workspace_bytes(1, 1, 1, 1, -1, ctypes.byref(out)) == _lib.DBF_ERR_INVALID_ARG


# Fake, never-dereferenced addresses: validation rejects before any launch.
A = 0x10000  # 16-byte aligned
MIS = 0x10002  # misaligned


@pytest.mark.parametrize("args,want", [
    ((0, 64, 128, A), _lib.DBF_ERR_INVALID_ARG),
    ((A, 64, 128, 0), _lib.DBF_ERR_INVALID_ARG),
    ((A, 0, 128, A + 4096), _lib.DBF_ERR_INVALID_ARG),
    ((A, 64, -3, A + 4096), _lib.DBF_ERR_INVALID_ARG),
    ((A, (1 << 30) + 1, 128, A + 4096), _lib.DBF_ERR_INVALID_ARG),
    ((A, 64, 128, A), _lib.DBF_ERR_INVALID_ARG),  # in place
    ((MIS, 64, 128, A), _lib.DBF_ERR_ALIGNMENT),
    ((A, 64, 128, MIS), _lib.DBF_ERR_ALIGNMENT),
])
def test_transpose_errors(args, want):
    src, rows, cols, dst = args
    assert L.dbf_transpose_signs(ctypes.c_void_p(src), rows, cols, ctypes.c_void_p(dst),
                                 None) == want


def _fwd(**kw):
    a = dict(x=A, ldx=64, B1=A, B2=A, alpha=A, beta=A, gamma=A, N=32, R=16, M=64, ell=1, T=4,
             y=A, ldy=32, y_type=_lib.DBF_F16, flags=0, ws=A, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.dbf_forward(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(N=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(R=-1), _lib.DBF_ERR_INVALID_ARG),
    (dict(M=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(ell=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(T=-1), _lib.DBF_ERR_INVALID_ARG),
    (dict(N=(1 << 30) + 1), _lib.DBF_ERR_INVALID_ARG),
    (dict(T=(1 << 30) + 1), _lib.DBF_ERR_INVALID_ARG),
    (dict(x=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(y=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(B1=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(gamma=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.DBF_ERR_INVALID_ARG),
    (dict(ldy=31), _lib.DBF_ERR_INVALID_ARG),
    (dict(y_type=_lib.DBF_I8), _lib.DBF_ERR_INVALID_ARG),
    (dict(y_type=7), _lib.DBF_ERR_INVALID_ARG),
    (dict(flags=64), _lib.DBF_ERR_INVALID_ARG),
    (dict(flags=_lib.DBF_PATH_GEMV | _lib.DBF_PATH_MFMA), _lib.DBF_ERR_INVALID_ARG),
    (dict(flags=128), _lib.DBF_ERR_INVALID_ARG),
    (dict(x=MIS), _lib.DBF_ERR_ALIGNMENT),
    (dict(y=MIS), _lib.DBF_ERR_ALIGNMENT),
    (dict(ldx=66), _lib.DBF_ERR_ALIGNMENT),
    (dict(ldy=36), _lib.DBF_ERR_ALIGNMENT),
    (dict(B2=MIS), _lib.DBF_ERR_ALIGNMENT),
    (dict(alpha=A + 1), _lib.DBF_ERR_ALIGNMENT),
    (dict(ws=None), _lib.DBF_ERR_WORKSPACE),
    (dict(ws_bytes=16), _lib.DBF_ERR_WORKSPACE),
])
def test_forward_rejects(kw, want):
    assert _fwd(**kw) == want


def test_forward_T0_is_noop():
    assert _fwd(T=0, x=None, y=None, ws=None, ws_bytes=0) == _lib.DBF_OK


def test_forward_fp32_ldy_multiple_of_4_ok_for_validation():
    # ldy = 36 is fine for fp32 output; with a too-small workspace the call
    # stops at the workspace check, proving the stride check passed.
    assert _fwd(ldy=36, y_type=_lib.DBF_F32, ws_bytes=16) == _lib.DBF_ERR_WORKSPACE


def _multi(**kw):
    a = dict(x=A, ldx=64, T=4, ids=A, num_adapters=3, B1s=A, B2s=A, alphas=A, betas=A, gammas=A,
             N=32, R=16, M=64, ell=1, y=A, ldy=32, y_type=_lib.DBF_F16, flags=0, ws=A,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.dbf_forward_multi_adapter(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(num_adapters=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(ids=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(B1s=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(gammas=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(N=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(ids=A + 2), _lib.DBF_ERR_ALIGNMENT),
    (dict(B2s=A + 4), _lib.DBF_ERR_ALIGNMENT),
    (dict(ws_bytes=0), _lib.DBF_ERR_WORKSPACE),
])
def test_multi_rejects(kw, want):
    assert _multi(**kw) == want


def test_pack_rejects():
    assert L.dbf_pack_signs(A, _lib.DBF_I8, 0, 4, 4, A, None) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_pack_signs(A, _lib.DBF_I8, 4, 4, 3, A, None) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_pack_signs(A, 9, 4, 4, 4, A, None) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_pack_signs(None, _lib.DBF_F16, 4, 4, 4, A, None) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_pack_signs(A, _lib.DBF_F32, 4, 4, 4, MIS, None) == _lib.DBF_ERR_ALIGNMENT
    assert L.dbf_unpack_signs(MIS, 4, 4, A, 4, None) == _lib.DBF_ERR_ALIGNMENT
    assert L.dbf_unpack_signs(A, 4, 4, A, 3, None) == _lib.DBF_ERR_INVALID_ARG


def _bwd(**kw):
    a = dict(x=A, ldx=64, g=A, ldg=32, B1=A, B2=A, B1t=A, B2t=A, alpha=A, beta=A, gamma=A,
             N=32, R=16, M=64, ell=1, T=4, dx=A, lddx=64, dx_type=_lib.DBF_F16, dalpha=A,
             dbeta=A, dgamma=A, dS1=None, dS2=None, H1=None, H2=None, tau=0.0, dH1=None,
             dH2=None, ws=A, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.dbf_backward(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(N=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(T=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(ell=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(M=(1 << 30) + 1), _lib.DBF_ERR_INVALID_ARG),
    (dict(ell=1 << 20, T=1 << 12), _lib.DBF_ERR_INVALID_ARG),
    (dict(g=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(B2t=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(dgamma=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(dx=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(H1=A), _lib.DBF_ERR_INVALID_ARG),            # latent without its output
    (dict(dH2=A), _lib.DBF_ERR_INVALID_ARG),           # output without its latent
    (dict(H1=A, dH1=A, tau=0.0), _lib.DBF_ERR_INVALID_ARG),
    (dict(H1=A, dH1=A, tau=-1.0), _lib.DBF_ERR_INVALID_ARG),
    (dict(H1=A, dH1=A, tau=float("inf")), _lib.DBF_ERR_INVALID_ARG),
    (dict(dx_type=_lib.DBF_I8), _lib.DBF_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.DBF_ERR_INVALID_ARG),
    (dict(ldg=31), _lib.DBF_ERR_INVALID_ARG),
    (dict(lddx=10), _lib.DBF_ERR_INVALID_ARG),
    (dict(x=MIS), _lib.DBF_ERR_ALIGNMENT),
    (dict(ldg=36), _lib.DBF_ERR_ALIGNMENT),
    (dict(B1t=MIS), _lib.DBF_ERR_ALIGNMENT),
    (dict(beta=A + 1), _lib.DBF_ERR_ALIGNMENT),
    (dict(dS1=A + 2), _lib.DBF_ERR_ALIGNMENT),
    (dict(dx=A + 2, dx_type=_lib.DBF_F32), _lib.DBF_ERR_ALIGNMENT),
    (dict(ws=None), _lib.DBF_ERR_WORKSPACE),
    (dict(ws_bytes=1024), _lib.DBF_ERR_WORKSPACE),
    (dict(ws=MIS), _lib.DBF_ERR_ALIGNMENT),
])
def test_backward_rejects(kw, want):
    assert _bwd(**kw) == want


def test_backward_workspace_bytes():
    out = ctypes.c_size_t(0)
    assert L.dbf_backward_workspace_bytes(32, 16, 64, 1, 4, ctypes.byref(out)) == _lib.DBF_OK
    assert out.value > 0
    small = out.value
    assert L.dbf_backward_workspace_bytes(32, 16, 64, 2, 300, ctypes.byref(out)) == _lib.DBF_OK
    assert out.value > small
    for bad in ((0, 16, 64, 1, 4), (32, 16, 64, 0, 4), (32, 16, 64, 1, 0)):
        assert L.dbf_backward_workspace_bytes(*bad, ctypes.byref(out)) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_backward_workspace_bytes(32, 16, 64, 1, 4, None) == _lib.DBF_ERR_INVALID_ARG


def _fac(**kw):
    a = dict(W=A, N=64, M=48, ldw=48, k=8, omega=A, X0=None, Y0=None, outer=1, admm_iters=2,
             power_iters=4, rho0=1.0, S1=A, S2=A, alpha=A, beta=A, gamma=A, rel_err=None, ws=A,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.dbf_factorize(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(N=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(k=-1), _lib.DBF_ERR_INVALID_ARG),
    (dict(M=(1 << 30) + 1), _lib.DBF_ERR_INVALID_ARG),
    (dict(W=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(S2=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(gamma=None), _lib.DBF_ERR_INVALID_ARG),
    (dict(omega=None), _lib.DBF_ERR_INVALID_ARG),             # no start at all
    (dict(omega=None, X0=A), _lib.DBF_ERR_INVALID_ARG),       # half a start
    (dict(X0=A), _lib.DBF_ERR_INVALID_ARG),
    (dict(ldw=40), _lib.DBF_ERR_INVALID_ARG),
    (dict(outer=-1), _lib.DBF_ERR_INVALID_ARG),
    (dict(admm_iters=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(power_iters=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(rho0=0.0), _lib.DBF_ERR_INVALID_ARG),
    (dict(rho0=float("nan")), _lib.DBF_ERR_INVALID_ARG),
    (dict(W=A + 2), _lib.DBF_ERR_ALIGNMENT),
    (dict(omega=A + 1), _lib.DBF_ERR_ALIGNMENT),
    (dict(beta=A + 1), _lib.DBF_ERR_ALIGNMENT),
    (dict(ws=None), _lib.DBF_ERR_WORKSPACE),
    (dict(ws_bytes=4096), _lib.DBF_ERR_WORKSPACE),
    (dict(ws=MIS), _lib.DBF_ERR_ALIGNMENT),
])
def test_factorize_rejects(kw, want):
    assert _fac(**kw) == want


def test_factorize_workspace_bytes():
    out = ctypes.c_size_t(0)
    assert L.dbf_factorize_workspace_bytes(64, 48, 8, ctypes.byref(out)) == _lib.DBF_OK
    small = out.value
    assert L.dbf_factorize_workspace_bytes(640, 480, 80, ctypes.byref(out)) == _lib.DBF_OK
    assert out.value > small > 0
    assert L.dbf_factorize_workspace_bytes(0, 48, 8, ctypes.byref(out)) == _lib.DBF_ERR_INVALID_ARG
    assert L.dbf_factorize_workspace_bytes(64, 48, 8, None) == _lib.DBF_ERR_INVALID_ARG


def _grp(**kw):
    arr = (ctypes.c_void_p * 3)(A, A, A)
    a = dict(x=A, ldx=64, T=4, J=3, B1s=arr, B2s=arr, alphas=arr, betas=arr, gammas=arr, N=32,
             R=16, M=64, ell=1, y=A, ldy=32, ys=32 * 4, y_type=_lib.DBF_F16, flags=0, ws=A,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.dbf_forward_grouped(*a.values())


def test_grouped_rejects():
    arr0 = (ctypes.c_void_p * 3)(A, None, A)
    mis = (ctypes.c_void_p * 3)(A, MIS, A)
    odd = (ctypes.c_void_p * 3)(A, A + 1, A)
    assert _grp(J=0) == _lib.DBF_ERR_INVALID_ARG
    assert _grp(J=9) == _lib.DBF_ERR_INVALID_ARG
    assert _grp(B1s=None) == _lib.DBF_ERR_INVALID_ARG
    assert _grp(B2s=arr0) == _lib.DBF_ERR_INVALID_ARG
    assert _grp(B1s=mis) == _lib.DBF_ERR_ALIGNMENT
    assert _grp(gammas=odd) == _lib.DBF_ERR_ALIGNMENT
    assert _grp(ys=32 * 3) == _lib.DBF_ERR_INVALID_ARG      # outputs would overlap
    assert _grp(ys=32 * 4 + 4) == _lib.DBF_ERR_ALIGNMENT    # 8 bytes off 16
    assert _grp(ldx=63) == _lib.DBF_ERR_INVALID_ARG
    assert _grp(ws_bytes=1024) == _lib.DBF_ERR_WORKSPACE
    assert _grp(T=0) == _lib.DBF_OK  # no-op
    out = ctypes.c_size_t(0)
    assert L.dbf_grouped_workspace_bytes(32, 16, 64, 1, 4, 3, ctypes.byref(out)) == _lib.DBF_OK
    one = ctypes.c_size_t(0)
    assert L.dbf_grouped_workspace_bytes(32, 16, 64, 1, 4, 1, ctypes.byref(one)) == _lib.DBF_OK
    assert out.value == 3 * one.value
    assert L.dbf_grouped_workspace_bytes(32, 16, 64, 1, 4, 9, ctypes.byref(out)) == \
        _lib.DBF_ERR_INVALID_ARG


def test_rank_and_plan_match_the_definition():
    import double_binary_rank_amd as dbf
    """The library's host planning equals the oracle's definitions: the rank
    for a bits budget, and the channels kept by non-uniform pruning."""
    import numpy as np
    import oracle
    for (N, M) in ((4096, 4096), (14336, 4096), (300, 17)):
        for bpw in (0.3, 1.0, 1.5, 2.0, 2.7):
            assert dbf.rank_for_bits(N, M, bpw) == oracle.rank_for_bits(N, M, bpw)
    rng = np.random.default_rng(60)
    shapes = [(40, 12, 30), (17, 20, 9), (64, 7, 64), (5, 30, 11)]
    imps = [rng.random(R) for (_, R, _) in shapes]
    imps[1][3] = imps[0][5]  # a tie across layers
    full = sum(dbf.layer_bits(*s) for s in shapes)
    for frac in (1.0, 0.9, 0.6, 0.3, 0.0):
        got = dbf.plan_channels(shapes, imps, frac * full)
        want = oracle.prune_channels(shapes, imps, frac * full)
        assert all(np.array_equal(g, w) for g, w in zip(got, want))


def test_planner_importance_and_gather():
    """The host planner's channel importance equals the oracle's definition,
    and its channel gather takes the kept columns of S1, rows of S2 and
    entries of beta, rejecting unsorted, repeated or out-of-range indices."""
    import numpy as np
    import oracle
    from double_binary_rank_amd import planner
    rng = np.random.default_rng(61)
    a, b, g = (rng.standard_normal((1, n)).astype(np.float16) for n in (37, 11, 23))
    assert np.allclose(planner.channel_importance(a, b, g), oracle.channel_importance(a, b, g),
                       rtol=1e-13, atol=0)
    with pytest.raises(ValueError):
        planner.channel_importance(np.ones((2, 37)), np.ones((2, 11)), np.ones((2, 23)))
    S1 = rng.choice([-1, 1], size=(9, 11)).astype(np.int8)
    S2 = rng.choice([-1, 1], size=(11, 7)).astype(np.int8)
    beta = rng.standard_normal((2, 11)).astype(np.float16)
    keep = np.array([0, 3, 4, 10])
    S1k, S2k, bk = planner.select_channels(S1, S2, beta, keep)
    for r_new, r in enumerate(keep):
        assert np.array_equal(S1k[:, r_new], S1[:, r])
        assert np.array_equal(S2k[r_new], S2[r])
        assert np.array_equal(bk[:, r_new], beta[:, r])
    for bad in ([], [3, 1], [2, 2], [-1, 4], [0, 11]):
        with pytest.raises(ValueError):
            planner.select_channels(S1, S2, beta, bad)


def _fwd_na(**kw):
    a = dict(x=A, ldx=64, B1=A, B2=A, alpha=A, beta=A, gamma=A, N=32, R=16, M=64, ell=1, T=4,
             y=A, ldy=32, y_type=_lib.DBF_F16, flags=0, stream=None)
    a.update(kw)
    return L.dbf_forward_no_alloc(*a.values())


@pytest.mark.parametrize("kw,want", [
    (dict(N=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(ell=0), _lib.DBF_ERR_INVALID_ARG),
    (dict(T=-1), _lib.DBF_ERR_INVALID_ARG),
    (dict(M=(1 << 30) + 1), _lib.DBF_ERR_INVALID_ARG),
    # workspaces beyond the static array are refused before anything else
    (dict(N=14336, R=6368, M=4096, T=4096, ldx=4096, ldy=14336), _lib.DBF_ERR_TOO_LARGE),
    (dict(N=4096, R=64, M=4096, ell=2, T=2048, ldx=4096, ldy=4096), _lib.DBF_ERR_TOO_LARGE),
])
def test_forward_no_alloc_rejects(kw, want):
    assert _fwd_na(**kw) == want


def test_forward_no_alloc_T0_is_noop():
    assert _fwd_na(T=0, x=None, y=None) == _lib.DBF_OK


def test_no_alloc_limit_matches_header():
    import re
    with open(os.path.join(ROOT, "include", "dbf.h")) as f:
        h = f.read()
    m = re.search(r"#define DBF_NO_ALLOC_SCRATCH_BYTES \(\(\(size_t\)(\d+)\) << (\d+)\)", h)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NO_ALLOC_SCRATCH_BYTES
    # the decode and T = 256 shapes of the workloads fit
    for shape in ((4096, 2048, 4096, 1, 256), (14336, 6368, 4096, 1, 256),
                  (4096, 6368, 14336, 1, 256), (4096, 64, 4096, 1, 8)):
        assert L.dbf_workspace_bytes(*shape, ctypes.byref(ctypes.c_size_t())) == 0
        assert _lib.workspace_bytes(*shape) <= _lib.NO_ALLOC_SCRATCH_BYTES


def test_binding_row_major_and_checks():
    """The binding's layout and argument checks (host logic, no device)."""
    import torch
    from double_binary_rank_amd import api
    x = torch.zeros(5, 12, dtype=torch.float16)
    assert api._row_major(x, "x") == 12
    assert api._row_major(torch.zeros(5, 16)[:, :12], "x") == 16      # padded rows
    assert api._row_major(torch.zeros(1, 12)[:, :12], "x") == 12
    assert api._row_major(torch.zeros(4, 16)[1:2, :8], "x") == 16     # one row
    assert api._row_major(torch.zeros(8).as_strided((1, 8), (1, 1)), "x") == 8  # any row stride
    assert api._row_major(torch.zeros(3, 8)[:, :1], "x") == 8        # one column: any inner stride
    with pytest.raises(ValueError):
        api._row_major(torch.zeros(8, 3).t(), "x")                     # inner stride 3
    with pytest.raises(ValueError):
        api._row_major(torch.zeros(2, 3, 4), "x")
    with pytest.raises(ValueError):
        api._need(x, "x", torch.float16)                               # not a device tensor
    with pytest.raises(ValueError):
        api._need(None, "x", torch.float16)
    assert api._flags(False, None) == 0
    assert api._flags(True, None) == 1
    assert api._flags(False, "gemv", ["prep", "stage2"]) == 2 | 8 | 32
    with pytest.raises(ValueError):
        api._flags(False, "nope")
    with pytest.raises(ValueError):
        api._flags(False, None, "stage3")
