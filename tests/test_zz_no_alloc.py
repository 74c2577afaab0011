"""dbf_forward_no_alloc: the forward product with the library's static
per-GPU workspace, for callers that cannot allocate device memory.  Checked
through the C ABI against dbf_forward (which takes a caller workspace) on
consecutive calls, the second one smaller, so the second call runs on what
the first left in the shared array."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _dbf():
    import double_binary_rank_amd as dbf
    return dbf


def _H():
    import gpu_helpers
    return gpu_helpers


CASES = [
    # (N, R, M, T, integer, y_f32): large-T path first, then smaller calls
    (1024, 512, 768, 200, True, True),
    (1024, 512, 768, 3, True, True),
    (520, 136, 264, 64, False, False),
    (520, 136, 264, 1, False, True),
]


def _run_pair(N, R, M, T, integer, y_f32, seed):
    dbf = _dbf()
    H = _H()
    kind = dict(alpha="ones", beta="ones", gamma="ones", x_kind="int3") if integer else {}
    L = synth.make_layer(N, R, M, 1, T, seed=seed, **kind)
    pl = H.upload(L)
    x = H.to_dev_rows(L.x)
    ydt = torch.float32 if y_f32 else torch.float16
    y_ref = pl.forward(x, y_dtype=ydt)
    y_na = H.empty_rows(T, N, ydt)
    dbf.dbf_forward_no_alloc(x, pl.B1, pl.B2, pl.alpha, pl.beta, pl.gamma, N, R, M, y_na)
    torch.cuda.synchronize()
    got = y_na.float().cpu().numpy().astype(np.float64)
    ref = y_ref.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)  # same kernels, same arithmetic
    want = oracle.forward(L.x, L.S1, L.S2, L.alpha, L.beta, L.gamma)
    if integer:
        assert np.array_equal(got, want.astype(np.float32).astype(np.float64))
    else:
        assert oracle.max_norm_error(got, want) <= 2e-3


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3)])
def test_no_alloc_matches_forward_twice(first, second):
    """Two calls in a row, the second with fewer tokens."""
    for j, c in enumerate((first, second)):
        _run_pair(*CASES[c], seed=7100 + 10 * first + j)


def test_no_alloc_rejects_oversized_call():
    """A call whose workspace would exceed the static array is refused on
    the host, before any launch, with its own status."""
    dbf = _dbf()
    lib = dbf._lib
    need = dbf.dbf_workspace_bytes(14336, 6368, 4096, 1, 4096)
    assert need > lib.NO_ALLOC_SCRATCH_BYTES
    x = torch.zeros((4096, 4096), dtype=torch.float16, device="cuda")
    y = torch.zeros((4096, 14336), dtype=torch.float16, device="cuda")
    b = torch.zeros(16, dtype=torch.uint8, device="cuda")
    s = torch.ones((1, 16384), dtype=torch.float16, device="cuda")
    with pytest.raises(lib.DbfError) as e:
        dbf.dbf_forward_no_alloc(x, b, b, s, s, s, 14336, 6368, 4096, y)
    assert e.value.status == lib.DBF_ERR_TOO_LARGE
