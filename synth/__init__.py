"""Seeded synthetic inputs for the double-binary-factorised (DBF) product.

This module only draws random numbers in a fixed order and rounds them to the
storage types (int8 signs, fp16 scales and activations). It holds none of the
method's arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``double_binary_rank_amd``) can be fed from it without sharing any code.

Shapes and value distributions stand in for the layers the pages evaluate on
(Llama-2/3 hidden size 4096, MLP width 14336); no weights or datasets are used.
The sign matrices are i.i.d. Bernoulli(0.5) in {-1, +1}, the storage the pages
describe for B1/B2 (LoRDBA summary, section 2 "Arquitectura Central"; DBF
summary, section 2 "Formulacion Matematica": A and B are sign matrices, a, m, b
are fp16 scale vectors).

Draw order per layer (fixed): S2, S1, gamma, beta, alpha, x, outlier channels,
ids.  Every real value is drawn in float64 and rounded to fp16 with numpy's
round-to-nearest-even conversion.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Layer",
    "MultiAdapterBatch",
    "CONFIGS",
    "config_seed",
    "make_signs",
    "make_layer",
    "make_config_layer",
    "make_multi_adapter",
    "zipf_ids",
]


@dataclasses.dataclass
class Layer:
    """One DBF layer plus a batch of activations.

    S1: int8 [N][R] in {-1,+1}; S2: int8 [R][M]; alpha [ell][N], beta [ell][R],
    gamma [ell][M] fp16; x fp16 [T][M].
    """

    S1: np.ndarray
    S2: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    gamma: np.ndarray
    x: np.ndarray

    @property
    def N(self) -> int:
        return self.S1.shape[0]

    @property
    def R(self) -> int:
        return self.S1.shape[1]

    @property
    def M(self) -> int:
        return self.S2.shape[1]

    @property
    def ell(self) -> int:
        return self.alpha.shape[0]

    @property
    def T(self) -> int:
        return self.x.shape[0]


@dataclasses.dataclass
class MultiAdapterBatch:
    """A batch of tokens, each routed to one of ``len(adapters)`` layers.

    adapters: list of Layer (their ``x`` fields are empty [0][M]);
    x fp16 [T][M]; ids int32 [T].
    """

    adapters: list
    x: np.ndarray
    ids: np.ndarray


def _f16(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def make_signs(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Bernoulli(0.5) signs in {-1, +1} as int8."""
    return (1 - 2 * rng.integers(0, 2, size=(rows, cols))).astype(np.int8)


# Scale / activation distributions, keyed by name.
def _scale_small_plus(rng, shape):  # 0.05 + |N(0,1)|*0.1
    return _f16(0.05 + np.abs(rng.standard_normal(shape)) * 0.1)


def _scale_abs002(rng, shape):  # |N(0,1)|*0.02
    return _f16(np.abs(rng.standard_normal(shape)) * 0.02)


def _scale_abs1(rng, shape):  # |N(0,1)|
    return _f16(np.abs(rng.standard_normal(shape)))


def _scale_lognormal(rng, shape):  # exp(N(-3, 0.5^2))
    return _f16(np.exp(rng.normal(-3.0, 0.5, size=shape)))


def _ones(rng, shape):
    return np.ones(shape, dtype=np.float16)


def _scale_pm12(rng, shape):  # uniform over {-2, -1, 1, 2}: products stay exact
    return rng.choice(np.array([-2.0, -1.0, 1.0, 2.0]), size=shape).astype(np.float16)


def _scale_pm1(rng, shape):  # uniform over {-1, 1}
    return rng.choice(np.array([-1.0, 1.0]), size=shape).astype(np.float16)


_SCALES = {
    "small_plus": _scale_small_plus,
    "abs002": _scale_abs002,
    "abs1": _scale_abs1,
    "lognormal": _scale_lognormal,
    "ones": _ones,
    "pm12": _scale_pm12,
    "pm1": _scale_pm1,
}


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    name: str
    N: int
    R: int
    M: int
    ell: int
    alpha: str
    beta: str
    gamma: str
    outlier_frac: float = 0.0  # fraction of input channels scaled x20


CONFIGS = {
    1: ConfigSpec("tiny", 256, 128, 256, 1, "small_plus", "small_plus", "small_plus"),
    2: ConfigSpec("lordba", 4096, 64, 4096, 1, "abs002", "abs1", "abs002"),
    3: ConfigSpec("attn_1bpw", 4096, 2048, 4096, 1, "lognormal", "lognormal", "lognormal"),
    4: ConfigSpec("mlp_up_2bpw", 14336, 6368, 4096, 1, "lognormal", "lognormal", "lognormal", 0.01),
    # down projection of the same MLP (N and M swapped)
    40: ConfigSpec("mlp_down_2bpw", 4096, 6368, 14336, 1, "lognormal", "lognormal", "lognormal", 0.01),
    5: ConfigSpec("multi_adapter", 4096, 64, 4096, 2, "abs002", "abs1", "abs002"),
}


def config_seed(config: int, T: int, integer: bool = False) -> int:
    """seed = 1000*config + T; the integer variant adds 7; the down projection
    of config 4 adds 1."""
    base = 4 if config == 40 else config
    s = 1000 * base + T
    if config == 40:
        s += 1
    if integer:
        s += 7
    return s


def make_layer(
    N: int,
    R: int,
    M: int,
    ell: int,
    T: int,
    seed: int,
    alpha: str = "small_plus",
    beta: str = "small_plus",
    gamma: str = "small_plus",
    x_kind: str = "normal",
    outlier_frac: float = 0.0,
    rng: np.random.Generator | None = None,
) -> Layer:
    """Draw one layer and T activation rows.

    x_kind: "normal" (N(0,1)), "int3" (uniform on the 7 integers -3..3),
    "none" (no activations drawn: x is [0][M]).
    """
    if rng is None:
        rng = np.random.default_rng(np.random.PCG64(seed))
    S2 = make_signs(rng, R, M)
    S1 = make_signs(rng, N, R)
    g = _SCALES[gamma](rng, (ell, M))
    b = _SCALES[beta](rng, (ell, R))
    a = _SCALES[alpha](rng, (ell, N))
    if x_kind == "normal":
        xf = rng.standard_normal((T, M))
    elif x_kind == "int3":
        xf = rng.integers(-3, 4, size=(T, M)).astype(np.float64)
    elif x_kind == "none":
        xf = np.zeros((0, M))
    else:
        raise ValueError(x_kind)
    if outlier_frac > 0.0:
        n_out = int(math.ceil(outlier_frac * M))
        chans = rng.choice(M, size=n_out, replace=False)
        xf[:, chans] *= 20.0
    return Layer(S1=S1, S2=S2, alpha=a, beta=b, gamma=g, x=_f16(xf))


def make_config_layer(config: int, T: int, integer: bool = False, seed: int | None = None) -> Layer:
    """The configuration's layer at T tokens.  ``integer`` selects the
    bit-exactness variant: x uniform on -3..3 and every scale exactly 1.0."""
    spec = CONFIGS[config]
    if seed is None:
        seed = config_seed(config, T, integer)
    if integer:
        return make_layer(spec.N, spec.R, spec.M, spec.ell, T, seed, "ones", "ones", "ones", "int3")
    return make_layer(
        spec.N, spec.R, spec.M, spec.ell, T, seed,
        spec.alpha, spec.beta, spec.gamma, "normal", spec.outlier_frac,
    )


def zipf_ids(rng: np.random.Generator, T: int, num: int, s: float = 1.1, sort: bool = True) -> np.ndarray:
    """Truncated Zipf(s) over ``num`` ids: P(rank k) proportional to k^-s for
    k = 1..num, rank k -> id k-1; optionally stable-sorted into segments."""
    k = np.arange(1, num + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    ids = rng.choice(num, size=T, p=p).astype(np.int32)
    if sort:
        ids = np.sort(ids, kind="stable")
    return ids


def make_multi_adapter(
    num_adapters: int = 64,
    N: int = 4096,
    R: int = 64,
    M: int = 4096,
    ell: int = 2,
    T: int = 2048,
    seed: int = 5000,
    alpha: str = "abs002",
    beta: str = "abs1",
    gamma: str = "abs002",
    x_kind: str = "normal",
    zipf_s: float = 1.1,
    sort: bool = True,
) -> MultiAdapterBatch:
    """Adapters drawn one after another (each in the per-layer order), then
    x, then the ids."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    adapters = [
        make_layer(N, R, M, ell, 0, seed, alpha, beta, gamma, "none", rng=rng)
        for _ in range(num_adapters)
    ]
    if x_kind == "normal":
        xf = rng.standard_normal((T, M))
    elif x_kind == "int3":
        xf = rng.integers(-3, 4, size=(T, M)).astype(np.float64)
    else:
        raise ValueError(x_kind)
    ids = zipf_ids(rng, T, num_adapters, zipf_s, sort)
    return MultiAdapterBatch(adapters=adapters, x=_f16(xf), ids=ids)
