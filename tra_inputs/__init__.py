"""Seeded synthetic q/k/v for spatiotemporal attention over a (T, H, W) token grid.

This module only *makes inputs*.  It holds none of the attention method's
arithmetic (no pooling, entropy, radius, masking or softmax), so that both the
fp64 CPU oracle and the HIP path can consume the very same bytes without
sharing any code of the method.

Layout of every tensor it returns: ``[heads][T][H][W][d]`` contiguous, batch 1,
values stored as bfloat16 bit patterns in ``numpy.uint16`` (round to nearest,
ties to even, from float32).

The workload recipe (the pages measure on trained video models that are not
available here; these synthetic tensors stand in for their activations):

* positions ``p = (t, y, x)`` in token units;
* per head, 16 random Fourier features of position,
  ``phi_raw_k(p) = sqrt(2) cos(w_k . p + b_k)`` with
  ``w_k = s_h * (g_t / ell_t, g_y / ell_s, g_x / ell_s)``, ``g ~ N(0, 1)^3``,
  ``b_k ~ U[0, 2 pi)``, projected to ``d`` by a ``16 x d`` matrix with entries
  ``N(0, 1/16)`` so that ``E|phi|^2 = d``;
* ``q = phi + sigma(p) eps_q`` and ``k = phi + sigma(p) eps_k`` (same ``phi``,
  independent standard-normal noise), ``v ~ N(0, 1)``;
* ``sigma`` maps: ``smooth`` (8 low-frequency Fourier features with length
  scales ``T/2, H/2, W/2``, min-max normalised to ``[0.1, 1.0]``),
  ``frames20`` (1.0 on a seeded 20 % of frames, 0.1 elsewhere) and
  ``bimodal80`` (1.0 where the smooth field exceeds its 80th percentile, 0.1
  elsewhere);
* per-head frequency scale ``s_h = 1``, or ``s_h ~ U[0.5, 4]`` when asked.

Every random stream is ``numpy.random.PCG64`` seeded by
``SeedSequence(seed, spawn_key=(config, head, stream))`` so that each head can
be regenerated on its own.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "TINY",
    "WAN13B_81F",
    "WAN13B_241F",
    "WAN14B_81F",
    "HUNYUAN_129F",
    "ELL_S",
    "ELL_T",
    "bf16_from_f32",
    "bf16_to_f32",
    "make_inputs",
    "make_workload_inputs",
    "aligned_qkv",
    "random_qkv",
    "sigma_map",
]

# Length scales of the Fourier position features, in tokens (space) and
# frames (time).  Fixed once by looking at the realised probe statistics of
# the 81-frame layer; see the design notes for the calibration record.
ELL_S = 8.0
ELL_T = 1.0

# stream ids inside a spawn key
_S_FEAT, _S_QN, _S_KN, _S_V, _S_SIGMA, _S_SCALE = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark/parity workload: grid, heads, head_dim and radius range."""

    name: str
    slug: str
    T: int
    H: int
    W: int
    heads: int
    d: int
    r_min: int
    r_max: int
    sigma: str = "smooth"
    head_scale: tuple | None = None  # (lo, hi) for s_h ~ U[lo, hi], else s_h = 1
    block: int = 64

    @property
    def N(self) -> int:
        return self.T * self.H * self.W


# Workload ids; an id is also the family of its inputs' random streams.
TINY, WAN13B_81F, WAN13B_241F, WAN14B_81F, HUNYUAN_129F = range(5)

WORKLOADS = {
    TINY: Workload("tiny T8xH8xW8, 1 head, d64", "tiny", 8, 8, 8, 1, 64, 0, 3),
    WAN13B_81F: Workload("Wan2.1-1.3B 480x832 81 frames (T21xH30xW52), 12 heads, d128",
                         "wan13b_81f", 21, 30, 52, 12, 128, 1, 8),
    WAN13B_241F: Workload("Wan2.1-1.3B 241 frames (T61xH30xW52), 12 heads, d128",
                          "wan13b_241f", 61, 30, 52, 12, 128, 1, 12, sigma="frames20"),
    WAN14B_81F: Workload("Wan2.1-14B 720x1280 81 frames (T21xH45xW80), 40 heads, d128",
                         "wan14b_81f", 21, 45, 80, 40, 128, 1, 10, head_scale=(0.5, 4.0)),
    HUNYUAN_129F: Workload("HunyuanVideo 720x1280 129 frames (T33xH45xW80), 24 heads, d128",
                           "hunyuan_129f", 33, 45, 80, 24, 128, 0, 16, sigma="bimodal80"),
}


def bf16_from_f32(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are assumed finite (the generator never makes NaN or Inf).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(h) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, family: int, head: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(family, head, stream))
    return np.random.Generator(np.random.PCG64(ss))


def _positions(T: int, H: int, W: int) -> np.ndarray:
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)


def _smooth_field(T: int, H: int, W: int, rng: np.random.Generator) -> np.ndarray:
    pos = _positions(T, H, W)
    ls = np.array([max(T / 2.0, 0.5), max(H / 2.0, 0.5), max(W / 2.0, 0.5)])
    g = rng.standard_normal((8, 3))
    b = rng.uniform(0.0, 2.0 * math.pi, size=8)
    u = np.cos(pos @ (g / ls).T + b).sum(axis=1)
    lo, hi = u.min(), u.max()
    if hi > lo:
        u = (u - lo) / (hi - lo)
    else:
        u = np.zeros_like(u)
    return u.reshape(T, H, W)


def sigma_map(T: int, H: int, W: int, kind: str, seed: int = 0, family: int = 0) -> np.ndarray:
    """Per-token noise level sigma(t, y, x) in [0.1, 1.0], shape (T, H, W)."""
    rng = _rng(seed, family, 0, _S_SIGMA)
    if kind == "smooth":
        return 0.1 + 0.9 * _smooth_field(T, H, W, rng)
    if kind == "frames20":
        n_hi = int(round(0.2 * T))
        frames = rng.choice(T, size=n_hi, replace=False)
        s = np.full((T, H, W), 0.1)
        s[frames] = 1.0
        return s
    if kind == "bimodal80":
        u = _smooth_field(T, H, W, rng)
        thr = np.percentile(u, 80.0)
        return np.where(u > thr, 1.0, 0.1)
    if kind == "none":
        return np.zeros((T, H, W))
    raise ValueError(f"unknown sigma map {kind!r}")


def make_inputs(T: int, H: int, W: int, heads: int, d: int, *, seed: int = 0,
                family: int = 0, sigma: str = "smooth", head_scale=None,
                ell_s: float = ELL_S, ell_t: float = ELL_T, heads_only=None):
    """Fourier-feature q/k plus N(0,1) v as bf16 bit patterns ``[heads][T][H][W][d]``.

    ``heads_only`` (a list of head indices) generates just those heads, in that
    order; each head's values are identical to the full generation's.
    """
    pos = _positions(T, H, W)
    sig = sigma_map(T, H, W, sigma, seed, family).reshape(-1, 1).astype(np.float32)
    if head_scale is not None:
        s_all = _rng(seed, family, 0, _S_SCALE).uniform(head_scale[0], head_scale[1], size=heads)
    else:
        s_all = np.ones(heads)
    hlist = list(range(heads)) if heads_only is None else list(heads_only)
    N = T * H * W
    q = np.empty((len(hlist), T, H, W, d), dtype=np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)
    inv_ell = np.array([1.0 / ell_t, 1.0 / ell_s, 1.0 / ell_s])
    for slot, h in enumerate(hlist):
        rf = _rng(seed, family, h, _S_FEAT)
        g = rf.standard_normal((16, 3))
        b = rf.uniform(0.0, 2.0 * math.pi, size=16)
        P = rf.standard_normal((16, d)) / 4.0  # N(0, 1/16)
        omega = s_all[h] * g * inv_ell
        phi_raw = math.sqrt(2.0) * np.cos(pos @ omega.T + b)
        phi = (phi_raw @ P).astype(np.float32)
        eq = _rng(seed, family, h, _S_QN).standard_normal((N, d), dtype=np.float32)
        ek = _rng(seed, family, h, _S_KN).standard_normal((N, d), dtype=np.float32)
        ev = _rng(seed, family, h, _S_V).standard_normal((N, d), dtype=np.float32)
        q[slot] = bf16_from_f32(phi + sig * eq).reshape(T, H, W, d)
        k[slot] = bf16_from_f32(phi + sig * ek).reshape(T, H, W, d)
        v[slot] = bf16_from_f32(ev).reshape(T, H, W, d)
    return q, k, v


def make_workload_inputs(wid: int, seed: int = 0, heads_only=None):
    """q, k, v for one of the named workloads in ``WORKLOADS``."""
    c = WORKLOADS[wid]
    return make_inputs(c.T, c.H, c.W, c.heads, c.d, seed=seed, family=wid,
                       sigma=c.sigma, head_scale=c.head_scale, heads_only=heads_only)


def aligned_qkv(T: int, H: int, W: int, heads: int, d: int, *, seed: int = 0,
                amp: float = 20.0, noise: float = 0.3, mixed_signs: bool = False):
    """q and k along one shared unit direction u, as bf16 bit patterns.

    k = amp u + noise e_k, and q = -amp u + noise e_q (every logit of every row
    strongly negative), or with mixed_signs each query token's sign drawn at
    random (rows of both signs side by side).  v ~ N(0, 1).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(98,))))
    shape = (heads, T, H, W, d)
    u = rng.standard_normal((heads, 1, 1, 1, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    sign = (rng.integers(0, 2, size=shape[:-1] + (1,)) * 2 - 1) if mixed_signs else -1.0
    q = sign * amp * u + noise * rng.standard_normal(shape)
    k = amp * u + noise * rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    return tuple(bf16_from_f32(a.astype(np.float32)) for a in (q, k, v))


def random_qkv(T: int, H: int, W: int, heads: int, d: int, *, seed: int = 0,
               scale: float = 1.0):
    """Plain i.i.d. N(0, scale^2) q, k, v as bf16 bit patterns (property tests)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(99,))))
    shape = (heads, T, H, W, d)
    out = []
    for _ in range(3):
        out.append(bf16_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)))
    return tuple(out)
