"""ctypes view of the C ABI in include/dbf.h (raw pointers and sizes only).

The library is the in-tree ``libdbf.so`` built by ``double_binary_rank_amd.build``.
There is no fallback: if it is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DBF_LIB_PATH names another build of the same library (a host-sanitized
# checking build); by default the in-tree libdbf.so
LIB_PATH = os.environ.get("DBF_LIB_PATH") or os.path.join(HERE, "libdbf.so")

DBF_OK = 0
DBF_ERR_INVALID_ARG = -1
DBF_ERR_ALIGNMENT = -2
DBF_ERR_WORKSPACE = -3
DBF_ERR_HIP = -4
DBF_ERR_TOO_LARGE = -5
NO_ALLOC_SCRATCH_BYTES = 32 << 20

DBF_I8 = 1
DBF_F16 = 2
DBF_F32 = 3

DBF_ACCUMULATE = 1
DBF_PATH_GEMV = 2
DBF_PATH_MFMA = 4
DBF_RUN_PREP = 8
DBF_RUN_STAGE1 = 16
DBF_RUN_STAGE2 = 32
MAX_DIM = 1 << 30

ABI_VERSION = 1

# every symbol include/dbf.h declares
EXPORTS = (
    "dbf_abi_version",
    "dbf_status_string",
    "dbf_packed_bytes",
    "dbf_pack_signs",
    "dbf_unpack_signs",
    "dbf_transpose_signs",
    "dbf_workspace_bytes",
    "dbf_forward",
    "dbf_forward_no_alloc",
    "dbf_forward_multi_adapter",
    "dbf_grouped_workspace_bytes",
    "dbf_forward_grouped",
    "dbf_backward_workspace_bytes",
    "dbf_backward",
    "dbf_factorize_workspace_bytes",
    "dbf_factorize",
)


class DbfError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def _hip_runtimes() -> set:
    """Paths of every libamdhip64 mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:  # pragma: no cover
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m double_binary_rank_amd.build`"
        )
    # PyTorch ships its own HIP runtime.  Load it first: the library then
    # binds to that same runtime (same soname), so stream handles and device
    # pointers from torch are valid in our launches.  Two runtimes in one
    # process would not share streams or contexts.
    import torch  # noqa: F401

    lib_ = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime mapped into the process: {sorted(runtimes)}")
    return lib_


lib = _load()

_i32, _i64, _u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t

lib.dbf_abi_version.restype = _i32
lib.dbf_abi_version.argtypes = []
lib.dbf_status_string.restype = ctypes.c_char_p
lib.dbf_status_string.argtypes = [_i32]
lib.dbf_packed_bytes.restype = _i32
lib.dbf_packed_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_sz)]
lib.dbf_pack_signs.restype = _i32
lib.dbf_pack_signs.argtypes = [_vp, _i32, _i64, _i64, _i64, _vp, _vp]
lib.dbf_unpack_signs.restype = _i32
lib.dbf_unpack_signs.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp]
lib.dbf_transpose_signs.restype = _i32
lib.dbf_transpose_signs.argtypes = [_vp, _i64, _i64, _vp, _vp]
lib.dbf_workspace_bytes.restype = _i32
lib.dbf_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, ctypes.POINTER(_sz)]
lib.dbf_forward.restype = _i32
lib.dbf_forward.argtypes = [
    _vp, _i64, _vp, _vp, _vp, _vp, _vp,  # x, ldx, B1, B2, alpha, beta, gamma
    _i64, _i64, _i64, _i32, _i64,  # N, R, M, ell, T
    _vp, _i64, _i32, _u32,  # y, ldy, y_type, flags
    _vp, _sz, _vp,  # ws, ws_bytes, stream
]
lib.dbf_forward_no_alloc.restype = _i32
lib.dbf_forward_no_alloc.argtypes = [
    _vp, _i64, _vp, _vp, _vp, _vp, _vp,  # x, ldx, B1, B2, alpha, beta, gamma
    _i64, _i64, _i64, _i32, _i64,  # N, R, M, ell, T
    _vp, _i64, _i32, _u32,  # y, ldy, y_type, flags
    _vp,  # stream
]
lib.dbf_forward_multi_adapter.restype = _i32
lib.dbf_forward_multi_adapter.argtypes = [
    _vp, _i64, _i64, _vp, _i32,  # x, ldx, T, ids, num_adapters
    _vp, _vp, _vp, _vp, _vp,  # B1s, B2s, alphas, betas, gammas (device tables)
    _i64, _i64, _i64, _i32,  # N, R, M, ell
    _vp, _i64, _i32, _u32,  # y, ldy, y_type, flags
    _vp, _sz, _vp,  # ws, ws_bytes, stream
]

lib.dbf_grouped_workspace_bytes.restype = _i32
lib.dbf_grouped_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
lib.dbf_forward_grouped.restype = _i32
lib.dbf_forward_grouped.argtypes = [
    _vp, _i64, _i64, _i32,  # x, ldx, T, num_layers
    _vp, _vp, _vp, _vp, _vp,  # B1s, B2s, alphas, betas, gammas (host pointer arrays)
    _i64, _i64, _i64, _i32,  # N, R, M, ell
    _vp, _i64, _i64, _i32, _u32,  # y, ldy, y_layer_stride, y_type, flags
    _vp, _sz, _vp,  # ws, ws_bytes, stream
]
lib.dbf_backward_workspace_bytes.restype = _i32
lib.dbf_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, ctypes.POINTER(_sz)]
lib.dbf_backward.restype = _i32
lib.dbf_backward.argtypes = [
    _vp, _i64, _vp, _i64,  # x, ldx, g, ldg
    _vp, _vp, _vp, _vp,  # B1, B2, B1t, B2t
    _vp, _vp, _vp,  # alpha, beta, gamma
    _i64, _i64, _i64, _i32, _i64,  # N, R, M, ell, T
    _vp, _i64, _i32,  # dx, lddx, dx_type
    _vp, _vp, _vp,  # dalpha, dbeta, dgamma
    _vp, _vp,  # dS1, dS2
    _vp, _vp, ctypes.c_float, _vp, _vp,  # H1, H2, tau, dH1, dH2
    _vp, _sz, _vp,  # ws, ws_bytes, stream
]

lib.dbf_factorize_workspace_bytes.restype = _i32
lib.dbf_factorize_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
lib.dbf_factorize.restype = _i32
lib.dbf_factorize.argtypes = [
    _vp, _i64, _i64, _i64, _i64,  # W, N, M, ldw, k
    _vp, _vp, _vp,  # omega, X0, Y0
    _i32, _i32, _i32, ctypes.c_float,  # outer, admm_iters, power_iters, rho0
    _vp, _vp, _vp, _vp, _vp, _vp,  # S1, S2, alpha, beta, gamma, rel_err
    _vp, _sz, _vp,  # ws, ws_bytes, stream
]


def status_string(status: int) -> str:
    return lib.dbf_status_string(status).decode()


def check(status: int, what: str) -> None:
    if status != DBF_OK:
        raise DbfError(status, what)


def abi_version() -> int:
    return lib.dbf_abi_version()


def packed_bytes(rows: int, cols: int) -> int:
    out = _sz(0)
    check(lib.dbf_packed_bytes(rows, cols, ctypes.byref(out)), "dbf_packed_bytes")
    return out.value


def workspace_bytes(N: int, R: int, M: int, ell: int, T: int) -> int:
    out = _sz(0)
    check(lib.dbf_workspace_bytes(N, R, M, ell, T, ctypes.byref(out)), "dbf_workspace_bytes")
    return out.value


def backward_workspace_bytes(N: int, R: int, M: int, ell: int, T: int) -> int:
    out = _sz(0)
    check(lib.dbf_backward_workspace_bytes(N, R, M, ell, T, ctypes.byref(out)),
          "dbf_backward_workspace_bytes")
    return out.value


def factorize_workspace_bytes(N: int, M: int, k: int) -> int:
    out = _sz(0)
    check(lib.dbf_factorize_workspace_bytes(N, M, k, ctypes.byref(out)),
          "dbf_factorize_workspace_bytes")
    return out.value


def grouped_workspace_bytes(N: int, R: int, M: int, ell: int, T: int, num_layers: int) -> int:
    out = _sz(0)
    check(lib.dbf_grouped_workspace_bytes(N, R, M, ell, T, num_layers, ctypes.byref(out)),
          "dbf_grouped_workspace_bytes")
    return out.value
