"""Thin PyTorch-side binding of the C ABI (include/dbf.h).

Argument marshalling only: tensors supply device pointers, strides and the
current HIP stream; every step of the product runs in the HIP library.
Function names follow the C entry points.  The offline planning of middle
widths (sizes, importances, the channel gather) is host numpy code in
``planner.py``; the methods here only move the factors to it and back.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import check, lib
from . import planner
from .planner import layer_bits, plan_channels, rank_for_bits  # noqa: F401  (re-exported)

__all__ = [
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
    "PackedLayer",
    "pointer_table",
    "rank_for_bits",
    "layer_bits",
    "plan_channels",
]

_DTYPE = {torch.int8: _lib.DBF_I8, torch.float16: _lib.DBF_F16, torch.float32: _lib.DBF_F32}


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: int | None = None) -> int:
    """The HIP stream handle: the given stream's, else the current stream of
    ``device`` (the current device when None).  Per call this is the host's
    hottest step, so the current stream is read as a raw handle without
    building a Stream object where torch offers that."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device() if device is None else device)
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _row_major(t: torch.Tensor, name: str) -> int:
    # a size-1 inner dimension may carry any stride
    sh, st = t.shape, t.stride()
    if len(sh) != 2 or (st[1] != 1 and sh[1] != 1):
        raise ValueError(f"{name} must be 2-D with unit inner stride")
    return max(st[0], sh[1]) if sh[0] == 1 else st[0]


def dbf_abi_version() -> int:
    return _lib.abi_version()


def dbf_status_string(status: int) -> str:
    return _lib.status_string(status)


def dbf_packed_bytes(rows: int, cols: int) -> int:
    return _lib.packed_bytes(rows, cols)


def dbf_workspace_bytes(N: int, R: int, M: int, ell: int, T: int) -> int:
    return _lib.workspace_bytes(N, R, M, ell, T)


def dbf_pack_signs(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Pack sign(src) (rows x cols, packed along cols).  Returns a uint8
    device tensor of dbf_packed_bytes(rows, cols) bytes (16-byte aligned)."""
    rows, cols = src.shape
    ld = _row_major(src, "src")
    nbytes = dbf_packed_bytes(rows, cols)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=src.device)
    check(lib.dbf_pack_signs(_ptr(src), _DTYPE[src.dtype], rows, cols, ld, _ptr(out),
                             _stream(stream)), "dbf_pack_signs")
    return out


def dbf_unpack_signs(packed: torch.Tensor, rows: int, cols: int, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.int8, device=packed.device)
    ld = _row_major(out, "out")
    check(lib.dbf_unpack_signs(_ptr(packed), rows, cols, _ptr(out), ld, _stream(stream)),
          "dbf_unpack_signs")
    return out


def dbf_transpose_signs(packed: torch.Tensor, rows: int, cols: int,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Packed signs of the cols x rows transpose of the packed rows x cols
    matrix ``packed``.  Returns a uint8 device tensor of
    dbf_packed_bytes(cols, rows) bytes."""
    if out is None:
        out = torch.empty(dbf_packed_bytes(cols, rows), dtype=torch.uint8, device=packed.device)
    check(lib.dbf_transpose_signs(_ptr(packed), rows, cols, _ptr(out), _stream(stream)),
          "dbf_transpose_signs")
    return out


_PHASE = {"prep": 8, "stage1": 16, "stage2": 32}


def _flags(accumulate: bool, path: str | None, phases=None) -> int:
    if path is None and phases is None:
        return _lib.DBF_ACCUMULATE if accumulate else 0
    f = _lib.DBF_ACCUMULATE if accumulate else 0
    if path == "gemv":
        f |= _lib.DBF_PATH_GEMV
    elif path == "mfma":
        f |= _lib.DBF_PATH_MFMA
    elif path not in (None, "auto"):
        raise ValueError(f"unknown path {path!r}")
    for ph in ([phases] if isinstance(phases, str) else (phases or ())):
        if ph not in _PHASE:
            raise ValueError(f"unknown phase {ph!r} (prep, stage1, stage2)")
        f |= _PHASE[ph]
    return f


def _padded_cols(N, dtype):
    # rows of 16-byte multiples, as the C ABI requires of ldy
    per = 16 // torch.empty((), dtype=dtype).element_size()
    return -(-N // per) * per


def _out(y, T, N, y_dtype, device):
    if y is None:
        y = torch.empty((T, _padded_cols(N, y_dtype)), dtype=y_dtype, device=device)[:, :N]
    return y, _row_major(y, "y")


def _ws(ws, N, R, M, ell, T, device):
    # (the library checks a given workspace's size itself)
    if ws is None:
        ws = torch.empty(max(dbf_workspace_bytes(N, R, M, ell, T), 16), dtype=torch.uint8,
                         device=device)
    return ws


def _need(t, name, dtype, contiguous=False):
    """The C ABI reads raw memory: reject a tensor whose dtype, device or
    layout it would misread."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check_scales(alpha, beta, gamma):
    _need(alpha, "alpha", torch.float16, contiguous=True)
    _need(beta, "beta", torch.float16, contiguous=True)
    _need(gamma, "gamma", torch.float16, contiguous=True)


def _check_out(y):
    if y is not None and y.dtype not in (torch.float16, torch.float32):
        raise TypeError(f"y must be float16 or float32, got {y.dtype}")


def _keep_alive(stream, *tensors):
    """Buffers made here for work on another stream than the current one:
    tell the caching allocator that stream uses them, so their memory is not
    reused before that work has run."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def dbf_forward(x: torch.Tensor, B1: torch.Tensor, B2: torch.Tensor, alpha: torch.Tensor,
                beta: torch.Tensor, gamma: torch.Tensor, N: int, R: int, M: int, *,
                y: torch.Tensor | None = None, y_dtype=torch.float16, accumulate: bool = False,
                path: str | None = None, ws: torch.Tensor | None = None,
                stream=None, phases=None) -> torch.Tensor:
    """y = sum_i diag(alpha_i) B1 diag(beta_i) B2 diag(gamma_i) x per token row.

    x [T][M] fp16; B1, B2 packed (dbf_pack_signs); alpha [ell][N],
    beta [ell][R], gamma [ell][M] fp16 contiguous.  ``phases`` (a name or a
    list of "prep", "stage1", "stage2") runs only those phases
    (DBF_RUN_PREP / DBF_RUN_STAGE1 / DBF_RUN_STAGE2); None runs all."""
    _need(x, "x", torch.float16)
    _need(B1, "B1", None)
    _need(B2, "B2", None)
    _check_scales(alpha, beta, gamma)
    _check_out(y)
    T = x.shape[0]
    ell = alpha.shape[0] if alpha.dim() == 2 else 1
    ldx = _row_major(x, "x")
    made_y, made_ws = y is None, ws is None
    y, ldy = _out(y, T, N, y_dtype, x.device)
    ws = _ws(ws, N, R, M, ell, T, x.device)
    yt = _DTYPE[y.dtype]
    check(lib.dbf_forward(_ptr(x), ldx, _ptr(B1), _ptr(B2), _ptr(alpha), _ptr(beta), _ptr(gamma),
                          N, R, M, ell, T, _ptr(y), ldy, yt, _flags(accumulate, path, phases), _ptr(ws),
                          ws.nbytes, _stream(stream, x.get_device())),
          "dbf_forward")
    _keep_alive(stream, y if made_y else None, ws if made_ws else None)
    return y


def dbf_forward_no_alloc(x: torch.Tensor, B1: torch.Tensor, B2: torch.Tensor,
                         alpha: torch.Tensor, beta: torch.Tensor, gamma: torch.Tensor, N: int,
                         R: int, M: int, y: torch.Tensor, *, accumulate: bool = False,
                         path: str | None = None, stream=None) -> torch.Tensor:
    """dbf_forward with the library's static per-GPU workspace: the caller
    passes the output y [T][N] (fp16 or fp32) and nothing is allocated."""
    _need(x, "x", torch.float16)
    _need(B1, "B1", None)
    _need(B2, "B2", None)
    _check_scales(alpha, beta, gamma)
    _need(y, "y", None)
    _check_out(y)
    T = x.shape[0]
    ell = alpha.shape[0] if alpha.dim() == 2 else 1
    ldx, ldy = _row_major(x, "x"), _row_major(y, "y")
    check(lib.dbf_forward_no_alloc(_ptr(x), ldx, _ptr(B1), _ptr(B2), _ptr(alpha), _ptr(beta),
                                   _ptr(gamma), N, R, M, ell, T, _ptr(y), ldy, _DTYPE[y.dtype],
                                   _flags(accumulate, path), _stream(stream, x.get_device())),
          "dbf_forward_no_alloc")
    return y


def dbf_grouped_workspace_bytes(N: int, R: int, M: int, ell: int, T: int, num_layers: int) -> int:
    return _lib.grouped_workspace_bytes(N, R, M, ell, T, num_layers)


def dbf_forward_grouped(x: torch.Tensor, layers, *, y: torch.Tensor | None = None,
                        y_dtype=torch.float16, accumulate: bool = False, path: str | None = None,
                        ws: torch.Tensor | None = None, stream=None, phases=None) -> torch.Tensor:
    """The same-input layers ``layers`` (PackedLayer, equal shapes, 1..8 of
    them) on x [T][M]: returns y [J][T][N] (or writes the given y of that
    shape; with ``accumulate`` adds onto it)."""
    J = len(layers)
    p0 = layers[0]
    N, R, M, ell = p0.N, p0.R, p0.M, p0.ell
    _need(x, "x", torch.float16)
    for p in layers:
        _check_scales(p.alpha, p.beta, p.gamma)
    _check_out(y)
    T = x.shape[0]
    ldx = _row_major(x, "x")
    made_y, made_ws = y is None, ws is None
    if y is None:
        y = torch.empty((J, T, _padded_cols(N, y_dtype)), dtype=y_dtype, device=x.device)[:, :, :N]
    if y.dim() != 3 or y.shape[0] != J or y.stride(2) != 1:
        raise ValueError("y must be [layers][T][N] with unit inner stride")
    ldy, ys = y.stride(1), y.stride(0)
    if ws is None:
        ws = torch.empty(max(dbf_grouped_workspace_bytes(N, R, M, ell, T, J), 16),
                         dtype=torch.uint8, device=x.device)
    arr = lambda ts: (ctypes.c_void_p * J)(*[t.data_ptr() for t in ts])  # noqa: E731
    check(lib.dbf_forward_grouped(
        _ptr(x), ldx, T, J, arr([p.B1 for p in layers]), arr([p.B2 for p in layers]),
        arr([p.alpha for p in layers]), arr([p.beta for p in layers]),
        arr([p.gamma for p in layers]), N, R, M, ell, _ptr(y), ldy, ys, _DTYPE[y.dtype],
        _flags(accumulate, path, phases), _ptr(ws), ws.nbytes,
        _stream(stream)), "dbf_forward_grouped")
    _keep_alive(stream, y if made_y else None, ws if made_ws else None)
    return y


def dbf_backward_workspace_bytes(N: int, R: int, M: int, ell: int, T: int) -> int:
    return _lib.backward_workspace_bytes(N, R, M, ell, T)


def dbf_backward(x: torch.Tensor, g: torch.Tensor, B1: torch.Tensor, B2: torch.Tensor,
                 B1t: torch.Tensor, B2t: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                 gamma: torch.Tensor, N: int, R: int, M: int, *, dx_dtype=torch.float16,
                 sign_grads: bool = False, H1: torch.Tensor | None = None,
                 H2: torch.Tensor | None = None, tau: float | None = None,
                 ws: torch.Tensor | None = None, stream=None) -> dict:
    """Gradients of one layer given the output gradient g = dL/dy [T][N] for
    the input x [T][M] (fp16): dx [T][M] (dx_dtype), dalpha [ell][N], dbeta
    [ell][R], dgamma [ell][M] (fp32); with ``sign_grads`` also dS1 [N][R] and
    dS2 [R][M]; with fp32 latents H1 [N][R] / H2 [R][M] and a temperature tau,
    the straight-through gradients dH1 / dH2.  B1t and B2t are the packed
    transposes (``dbf_transpose_signs``)."""
    _need(x, "x", torch.float16)
    _need(g, "g", torch.float16)
    _check_scales(alpha, beta, gamma)
    T = x.shape[0]
    ell = alpha.shape[0] if alpha.dim() == 2 else 1
    dev = x.device
    ldx, ldg = _row_major(x, "x"), _row_major(g, "g")
    made_ws = ws is None
    dx = torch.empty((T, M), dtype=dx_dtype, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": dx, "dalpha": torch.empty((ell, N), **f32), "dbeta": torch.empty((ell, R), **f32),
           "dgamma": torch.empty((ell, M), **f32)}
    if sign_grads:
        out["dS1"] = torch.empty((N, R), **f32)
        out["dS2"] = torch.empty((R, M), **f32)
    for name, H, shape in (("dH1", H1, (N, R)), ("dH2", H2, (R, M))):
        if H is not None:
            if H.dtype != torch.float32 or tuple(H.shape) != shape or not H.is_contiguous():
                raise ValueError(f"{name[1:]} must be contiguous fp32 of shape {shape}")
            out[name] = torch.empty(shape, **f32)
    need = dbf_backward_workspace_bytes(N, R, M, ell, T)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    check(lib.dbf_backward(
        _ptr(x), ldx, _ptr(g), ldg, _ptr(B1), _ptr(B2), _ptr(B1t), _ptr(B2t), _ptr(alpha),
        _ptr(beta), _ptr(gamma), N, R, M, ell, T, _ptr(dx), M, _DTYPE[dx_dtype],
        _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dgamma"]), _ptr(out.get("dS1")),
        _ptr(out.get("dS2")), _ptr(H1), _ptr(H2), 0.0 if tau is None else float(tau),
        _ptr(out.get("dH1")), _ptr(out.get("dH2")), _ptr(ws), ws.nbytes,
        _stream(stream)), "dbf_backward")
    _keep_alive(stream, *out.values(), ws if made_ws else None)
    return out


def dbf_factorize_workspace_bytes(N: int, M: int, k: int) -> int:
    return _lib.factorize_workspace_bytes(N, M, k)


def dbf_factorize(W: torch.Tensor, k: int, omega: torch.Tensor | None = None, *, outer: int = 3,
                  admm_iters: int = 10, power_iters: int = 8, rho0: float = 1.0, start=None,
                  ws: torch.Tensor | None = None, stream=None) -> dict:
    """Double binary factorisation of the fp32 matrix W [N][M] at inner
    dimension k: returns S1 int8 [N][k], S2 int8 [k][M], alpha [1][N], beta
    [1][k], gamma [1][M] fp16 and rel_err (a 0-d fp32 device tensor).  omega
    [k][N] fp32 is the caller's Gaussian sketch for the start, or ``start`` =
    (X0, Y0) fp32 scaled sign matrices."""
    _need(W, "W", torch.float32)
    if omega is not None:
        _need(omega, "omega", torch.float32, contiguous=True)
    N, M = W.shape
    ldw = _row_major(W, "W")
    dev = W.device
    made_ws = ws is None
    out = {"S1": torch.empty((N, k), dtype=torch.int8, device=dev),
           "S2": torch.empty((k, M), dtype=torch.int8, device=dev),
           "alpha": torch.empty((1, N), dtype=torch.float16, device=dev),
           "beta": torch.empty((1, k), dtype=torch.float16, device=dev),
           "gamma": torch.empty((1, M), dtype=torch.float16, device=dev),
           "rel_err": torch.empty((), dtype=torch.float32, device=dev)}
    X0 = Y0 = None
    if start is not None:
        X0, Y0 = (_need(t, "start", torch.float32).contiguous() for t in start)
    if ws is None:
        ws = torch.empty(dbf_factorize_workspace_bytes(N, M, k), dtype=torch.uint8, device=dev)
    check(lib.dbf_factorize(
        _ptr(W), N, M, ldw, k, _ptr(omega), _ptr(X0), _ptr(Y0), outer, admm_iters, power_iters,
        float(rho0), _ptr(out["S1"]), _ptr(out["S2"]), _ptr(out["alpha"]), _ptr(out["beta"]),
        _ptr(out["gamma"]), _ptr(out["rel_err"]), _ptr(ws), ws.nbytes,
        _stream(stream)), "dbf_factorize")
    _keep_alive(stream, *out.values(), ws if made_ws else None, X0, Y0)
    return out


def pointer_table(tensors, device) -> torch.Tensor:
    """Device int64 array of the tensors' device addresses."""
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def dbf_forward_multi_adapter(x: torch.Tensor, ids: torch.Tensor, B1s: torch.Tensor,
                              B2s: torch.Tensor, alphas: torch.Tensor, betas: torch.Tensor,
                              gammas: torch.Tensor, num_adapters: int, N: int, R: int, M: int,
                              ell: int, *, y: torch.Tensor | None = None, y_dtype=torch.float16,
                              accumulate: bool = False, path: str | None = None,
                              ws: torch.Tensor | None = None, stream=None,
                              phases=None) -> torch.Tensor:
    """Token t uses adapter ids[t]; the five tables are device int64 arrays
    of per-adapter device pointers (see ``pointer_table``)."""
    _need(x, "x", torch.float16)
    _need(ids, "ids", torch.int32, contiguous=True)
    for name, t in (("B1s", B1s), ("B2s", B2s), ("alphas", alphas), ("betas", betas),
                    ("gammas", gammas)):
        _need(t, name, torch.int64, contiguous=True)
        if t.numel() < num_adapters:
            raise ValueError(f"{name} holds fewer than num_adapters pointers")
    if ids.numel() != x.shape[0]:
        raise ValueError("ids must hold one id per token row of x")
    _check_out(y)
    T = x.shape[0]
    ldx = _row_major(x, "x")
    made_y, made_ws = y is None, ws is None
    y, ldy = _out(y, T, N, y_dtype, x.device)
    ws = _ws(ws, N, R, M, ell, T, x.device)
    yt = _DTYPE[y.dtype]
    check(lib.dbf_forward_multi_adapter(
        _ptr(x), ldx, T, _ptr(ids), num_adapters, _ptr(B1s), _ptr(B2s), _ptr(alphas), _ptr(betas),
        _ptr(gammas), N, R, M, ell, _ptr(y), ldy, yt, _flags(accumulate, path, phases), _ptr(ws),
        ws.nbytes, _stream(stream)), "dbf_forward_multi_adapter")
    _keep_alive(stream, y if made_y else None, ws if made_ws else None)
    return y


@dataclass
class PackedLayer:
    """One layer's factors resident on the device: packed B1 (N x R) and
    B2 (R x M) plus fp16 scales [ell][*]."""

    B1: torch.Tensor
    B2: torch.Tensor
    alpha: torch.Tensor
    beta: torch.Tensor
    gamma: torch.Tensor
    N: int
    R: int
    M: int

    @property
    def ell(self) -> int:
        return self.alpha.shape[0]

    @classmethod
    def from_signs(cls, S1, S2, alpha, beta, gamma, device="cuda") -> "PackedLayer":
        """S1 [N][R], S2 [R][M] sign (or latent) arrays; scales [ell][*] fp16.
        Host arrays are uploaded, then packed on the device."""
        def dev(a, dtype=None):
            t = torch.as_tensor(a)
            if dtype is not None:
                t = t.to(dtype)
            return t.to(device).contiguous()

        s1, s2 = dev(S1), dev(S2)
        a, b, g = (dev(v, torch.float16) for v in (alpha, beta, gamma))
        if a.dim() == 1:
            a, b, g = a[None], b[None], g[None]
        B1 = dbf_pack_signs(s1)
        B2 = dbf_pack_signs(s2)
        return cls(B1, B2, a.contiguous(), b.contiguous(), g.contiguous(), s1.shape[0],
                   s1.shape[1], s2.shape[1])

    def forward(self, x: torch.Tensor, **kw) -> torch.Tensor:
        return dbf_forward(x, self.B1, self.B2, self.alpha, self.beta, self.gamma, self.N, self.R,
                           self.M, **kw)

    @classmethod
    def from_factorization(cls, f: dict) -> "PackedLayer":
        """The layer of a ``dbf_factorize`` result (signs packed here)."""
        return cls(dbf_pack_signs(f["S1"]), dbf_pack_signs(f["S2"]), f["alpha"], f["beta"],
                   f["gamma"], f["S1"].shape[0], f["S1"].shape[1], f["S2"].shape[1])

    def channel_importance(self):
        """Per middle channel r (ell = 1): |beta_r| ||alpha|| ||gamma|| (see
        ``planner.channel_importance``), from host copies of the scales; a
        host float64 array."""
        if self.ell != 1:
            raise ValueError("channel importance is defined for ell = 1")
        return planner.channel_importance(self.alpha.cpu().numpy(), self.beta.cpu().numpy(),
                                          self.gamma.cpu().numpy())

    def select_channels(self, keep) -> "PackedLayer":
        """The layer restricted to the middle channels ``keep`` (sorted
        indices): the signs are unpacked by the library, gathered on the
        host by ``planner.select_channels`` and packed again by the library
        (offline)."""
        S1 = dbf_unpack_signs(self.B1, self.N, self.R).cpu().numpy()
        S2 = dbf_unpack_signs(self.B2, self.R, self.M).cpu().numpy()
        S1k, S2k, bk = planner.select_channels(S1, S2, self.beta.cpu().numpy(), keep)
        dev = self.B1.device
        return PackedLayer(dbf_pack_signs(torch.from_numpy(S1k).to(dev)),
                           dbf_pack_signs(torch.from_numpy(S2k).to(dev)), self.alpha,
                           torch.from_numpy(bk).to(dev), self.gamma, self.N, S1k.shape[1],
                           self.M)

    def transposed_signs(self):
        """Packed S1^T (R x N) and S2^T (M x R), built once per layer."""
        if getattr(self, "_signs_t", None) is None:
            self._signs_t = (dbf_transpose_signs(self.B1, self.N, self.R),
                             dbf_transpose_signs(self.B2, self.R, self.M))
        return self._signs_t

    def backward(self, x: torch.Tensor, g: torch.Tensor, **kw) -> dict:
        """Gradients for the output gradient g of ``forward(x)``; see
        ``dbf_backward``."""
        B1t, B2t = self.transposed_signs()
        return dbf_backward(x, g, self.B1, self.B2, B1t, B2t, self.alpha, self.beta, self.gamma,
                            self.N, self.R, self.M, **kw)

    def transposed(self) -> "PackedLayer":
        """The layer of dW^T = sum_i diag(gamma_i) S2^T diag(beta_i) S1^T
        diag(alpha_i) (M outputs, N inputs): its forward maps an output
        gradient g [T][N] to g dW [T][M], the input gradient."""
        return PackedLayer(dbf_transpose_signs(self.B2, self.R, self.M),
                           dbf_transpose_signs(self.B1, self.N, self.R),
                           self.gamma, self.beta, self.alpha, self.M, self.R, self.N)
