"""Helpers for the GPU tests: upload seeded inputs, run the HIP path through
the C ABI, and a host-side model of the documented packed layout."""
from __future__ import annotations

import numpy as np
import torch

import double_binary_rank_amd as dbf


def pack_ref(S: np.ndarray) -> np.ndarray:
    """The packed words of sign(S) under the layout the library documents:
    units of 64 rows (4 tiles of 16) x 128 cols, 1 KB each, quad-major;
    in a unit, word 4*lam + h holds row lam%16 of tile h; with g = lam//16,
    slot s of that word is block col 32*(s//8) + 8*g + s%8 and sits at bit
    4*(s%8) + s//8; bit 1 means -1."""
    rows, cols = S.shape
    nq, nkb = -(-rows // 64), -(-cols // 128)
    words = np.zeros(nq * nkb * 256, dtype=np.uint64)
    r, k = np.nonzero(np.asarray(S) < 0)
    c = k % 128
    g = (c // 8) % 4
    s = 8 * (c // 32) + c % 8
    lam = 16 * g + (r % 16)
    idx = ((r // 64) * nkb + k // 128) * 256 + 4 * lam + (r % 64) // 16
    bit = 4 * (s % 8) + s // 8
    np.bitwise_or.at(words, idx, (np.uint64(1) << bit.astype(np.uint64)))
    return words.astype(np.uint32)


def to_dev(a, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def to_dev_rows(a, dtype=None, mult=8):
    """2-D device tensor whose row stride is padded to a multiple of ``mult``
    elements (the ABI wants 16-byte aligned rows); returns the [rows][cols]
    view."""
    a = np.asarray(a)
    rows, cols = a.shape
    ld = -(-max(cols, 1) // mult) * mult
    t = torch.zeros((rows, ld), dtype=dtype or torch.from_numpy(a[:0]).dtype, device="cuda")
    t[:, :cols] = to_dev(a, dtype)
    return t[:, :cols]


def empty_rows(rows, cols, dtype, mult=8):
    ld = -(-max(cols, 1) // mult) * mult
    return torch.empty((rows, ld), dtype=dtype, device="cuda")[:, :cols]


def upload(L) -> dbf.PackedLayer:
    return dbf.PackedLayer.from_signs(L.S1, L.S2, L.alpha, L.beta, L.gamma, device="cuda")


def run_layer(L, path=None, y_dtype=torch.float16, accumulate=False, y_init=None, pl=None):
    pl = pl or upload(L)
    x = to_dev_rows(L.x)
    y = empty_rows(L.T, L.N, y_dtype) if y_init is None else to_dev_rows(y_init)
    out = pl.forward(x, path=path, y_dtype=y_dtype, accumulate=accumulate, y=y)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


class DeviceAdapters:
    """Per-adapter packed factors plus the device pointer tables."""

    def __init__(self, adapters, entries=None):
        """``entries``: for each pointer-table entry, the index of the adapter
        it points to (default: one entry per adapter)."""
        self.layers = [upload(a) for a in adapters]
        dev = "cuda"
        tab = self.layers if entries is None else [self.layers[e] for e in entries]
        self.n_entries = len(tab)
        self.B1s = dbf.pointer_table([p.B1 for p in tab], dev)
        self.B2s = dbf.pointer_table([p.B2 for p in tab], dev)
        self.alphas = dbf.pointer_table([p.alpha for p in tab], dev)
        self.betas = dbf.pointer_table([p.beta for p in tab], dev)
        self.gammas = dbf.pointer_table([p.gamma for p in tab], dev)
        p0 = self.layers[0]
        self.N, self.R, self.M, self.ell = p0.N, p0.R, p0.M, p0.ell

    def forward(self, x, ids, **kw):
        return dbf.dbf_forward_multi_adapter(
            x, ids, self.B1s, self.B2s, self.alphas, self.betas, self.gammas, self.n_entries,
            self.N, self.R, self.M, self.ell, **kw)
