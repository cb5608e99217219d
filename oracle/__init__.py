"""fp64 CPU oracle for entropy-radius block-sparse spatiotemporal attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users.  The product path (the HIP library and
its Python binding) never imports, links or runs anything here, and the two
share no code.  See ``tra_oracle.c`` for what each function computes and the
passages of the pages it follows.

Every function takes and returns numpy arrays; q, k and v are bfloat16 bit
patterns (``uint16``) in ``[heads][T][H][W][d]`` layout.

Parity pins: every function here is checked in ``tests/test_oracle.py``
against brute force, closed forms, invariants or library routines; none is
"parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

RADIUS_INF = 2147483647

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tra_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, IEEE fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        lib.orc_radius.argtypes = [ctypes.c_double, I, I]
        lib.orc_radius.restype = I
        lib.orc_pool.argtypes = [P, I, I, I, I, I, I, P]
        lib.orc_pool.restype = I
        lib.orc_probe.argtypes = [P, P, I, I, I, I, I, I, I, I, P, P]
        lib.orc_probe.restype = I
        lib.orc_block_lists.argtypes = [P, I, I, I, I, I, L, P, P]
        lib.orc_block_lists.restype = I
        lib.orc_attention_rows.argtypes = [P, P, P, I, I, I, I, I, I, P, L, P, P]
        lib.orc_attention_rows.restype = I
        lib.orc_attention.argtypes = [P, P, P, I, I, I, I, I, I, P, P]
        lib.orc_attention.restype = I
        D = ctypes.c_double
        lib.orc_token_entropy_rows.argtypes = [P, P, I, I, I, I, I, I, L, P, P]
        lib.orc_token_entropy_rows.restype = I
        lib.orc_token_radius.argtypes = [P, I, I, I, I, D, D, P]
        lib.orc_token_radius.restype = I
        lib.orc_token_lists.argtypes = [P, I, I, I, I, I, D, I, D, L, P, L, P, P]
        lib.orc_token_lists.restype = I
        lib.orc_attention_lists_rows.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, L, L, P, P]
        lib.orc_sip_lists.argtypes = [P, P, P, I, I, I, I, I, I, D, D, L, P, P, P]
        lib.orc_sip_lists.restype = I
        lib.orc_attention_lists_rows.restype = I
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = I
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("q/k/v must be bfloat16 bit patterns (uint16)")
    return x


def _dims(x):
    heads, T, H, W, d = x.shape
    return heads, T, H, W, d


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def num_threads() -> int:
    return _load().orc_num_threads()


def grid_blocks(T: int, H: int, W: int, block: int = 64):
    """(nby, nbx, nb) of the tile grid."""
    s = int(round(block ** 0.5))
    nby = -(-H // s)
    nbx = -(-W // s)
    return nby, nbx, T * nby * nbx


def radius(h_norm: float, r_min: int, r_max: int) -> int:
    return _load().orc_radius(float(h_norm), int(r_min), int(r_max))


def pool(x, block: int = 64) -> np.ndarray:
    """Block means over real tokens, fp64 ``[heads][nb][d]``."""
    x = _u16(x)
    heads, T, H, W, d = _dims(x)
    nb = grid_blocks(T, H, W, block)[2]
    out = np.empty((heads, nb, d), dtype=np.float64)
    _check(_load().orc_pool(_ptr(x), T, H, W, heads, d, block, _ptr(out)), "pool")
    return out


def probe(q, k, r_min: int, r_max: int, block: int = 64):
    """(h_norm fp64 ``[heads][nb]``, radius int32 ``[heads][nb]``)."""
    q, k = _u16(q), _u16(k)
    heads, T, H, W, d = _dims(q)
    assert k.shape == q.shape
    nb = grid_blocks(T, H, W, block)[2]
    hn = np.empty((heads, nb), dtype=np.float64)
    r = np.empty((heads, nb), dtype=np.int32)
    _check(_load().orc_probe(_ptr(q), _ptr(k), T, H, W, heads, d, block, r_min, r_max,
                             _ptr(hn), _ptr(r)), "probe")
    return hn, r


def block_lists(radii, T: int, H: int, W: int, block: int = 64, maxcnt: int | None = None):
    """(idx int32 ``[heads][nb][maxcnt]`` with -1 past cnt, cnt int32 ``[heads][nb]``)."""
    radii = np.ascontiguousarray(radii, dtype=np.int32)
    heads, nb = radii.shape
    assert nb == grid_blocks(T, H, W, block)[2]
    if maxcnt is None:
        maxcnt = nb
    idx = np.full((heads, nb, maxcnt), -1, dtype=np.int32)
    cnt = np.empty((heads, nb), dtype=np.int32)
    _check(_load().orc_block_lists(_ptr(radii), T, H, W, heads, block, maxcnt, _ptr(idx), _ptr(cnt)),
           "block_lists")
    return idx, cnt


def attention(q, k, v, radii, block: int = 64) -> np.ndarray:
    """Masked softmax attention for every token, fp64 ``[heads][T][H][W][d]``."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    heads, T, H, W, d = _dims(q)
    radii = np.ascontiguousarray(radii, dtype=np.int32)
    out = np.empty((heads, T, H, W, d), dtype=np.float64)
    _check(_load().orc_attention(_ptr(q), _ptr(k), _ptr(v), T, H, W, heads, d, block,
                                 _ptr(radii), _ptr(out)), "attention")
    return out


def attention_rows(q, k, v, radii, rows, block: int = 64) -> np.ndarray:
    """Masked softmax attention for the rows ``head * N + token``, fp64 ``[len(rows)][d]``."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    heads, T, H, W, d = _dims(q)
    radii = np.ascontiguousarray(radii, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), dtype=np.float64)
    _check(_load().orc_attention_rows(_ptr(q), _ptr(k), _ptr(v), T, H, W, heads, d, block,
                                      _ptr(radii), rows.size, _ptr(rows), _ptr(out)), "attention_rows")
    return out


def dense_radii(heads: int, nb: int) -> np.ndarray:
    return np.full((heads, nb), RADIUS_INF, dtype=np.int32)


# ---------------------------------------------- token-level radius policy --

def token_entropy_rows(q, k, rows, block: int = 64) -> np.ndarray:
    """Entropy of the dense attention row of each ``head * N + token`` row, fp64."""
    q, k = _u16(q), _u16(k)
    heads, T, H, W, d = _dims(q)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    ent = np.empty(rows.size, dtype=np.float64)
    _check(_load().orc_token_entropy_rows(_ptr(q), _ptr(k), T, H, W, heads, d, block, rows.size,
                                          _ptr(rows), _ptr(ent)), "token_entropy_rows")
    return ent


def token_entropy(q, k, block: int = 64) -> np.ndarray:
    """Entropy of every token's dense attention row, fp64 ``[heads][T][H][W]``."""
    heads, T, H, W, d = _dims(q)
    ent = token_entropy_rows(q, k, np.arange(heads * T * H * W), block)
    return ent.reshape(heads, T, H, W)


def token_radius(ent, tau: float, gamma: float) -> np.ndarray:
    """Base radius of every token from its entropy ``[heads][T][H][W]``, fp64."""
    ent = np.ascontiguousarray(ent, dtype=np.float64)
    heads, T, H, W = ent.shape
    r0 = np.empty_like(ent)
    _check(_load().orc_token_radius(_ptr(ent), T, H, W, heads, float(tau), float(gamma), _ptr(r0)),
           "token_radius")
    return r0


def token_lists(r0, gamma: float, min_votes: int = 1, block: int = 64, rows=None,
                r2_scale: float = 1.0, maxcnt: int | None = None):
    """Voting lists of the ``head * nb + query block`` rows (all by default):
    (idx int32 ``[rows][maxcnt]`` with -1 past cnt, cnt int32 ``[rows]``)."""
    r0 = np.ascontiguousarray(r0, dtype=np.float64)
    heads, T, H, W = r0.shape
    nb = grid_blocks(T, H, W, block)[2]
    rows = np.arange(heads * nb) if rows is None else rows
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    maxcnt = nb if maxcnt is None else maxcnt
    idx = np.full((rows.size, maxcnt), -1, dtype=np.int32)
    cnt = np.empty(rows.size, dtype=np.int32)
    _check(_load().orc_token_lists(_ptr(r0), T, H, W, heads, block, float(gamma), int(min_votes),
                                   float(r2_scale), rows.size, _ptr(rows), maxcnt, _ptr(idx),
                                   _ptr(cnt)), "token_lists")
    return idx, cnt


def attention_lists_rows(q, k, v, idx, cnt, rows, block: int = 64, lw=None) -> np.ndarray:
    """Softmax attention of the ``head * N + token`` rows over explicit key-block
    lists ``idx[heads][nb][maxcnt]``, ``cnt[heads][nb]``, with optional per-entry
    log-weights ``lw`` (same shape as idx); fp64 ``[len(rows)][d]``."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    heads, T, H, W, d = _dims(q)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    maxcnt = idx.shape[-1]
    lwp = None
    if lw is not None:
        lw = np.ascontiguousarray(lw, dtype=np.float64)
        assert lw.shape == idx.shape
        lwp = _ptr(lw)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), dtype=np.float64)
    _check(_load().orc_attention_lists_rows(_ptr(q), _ptr(k), _ptr(v), T, H, W, heads, d, block,
                                            _ptr(idx), _ptr(cnt), lwp, maxcnt, rows.size,
                                            _ptr(rows), _ptr(out)), "attention_lists_rows")
    return out


def sip_lists(q, k, u, m: float, block: int = 64, pi_scale: float = 1.0):
    """Sampled key-block lists with log-weights: (idx int32, cnt int32, lw fp64),
    idx/lw ``[heads][nb][nb]`` (-1 / 0 past cnt), for uniforms ``u[heads][nb][nb]``."""
    q, k = _u16(q), _u16(k)
    heads, T, H, W, d = _dims(q)
    nb = grid_blocks(T, H, W, block)[2]
    u = np.ascontiguousarray(u, dtype=np.float64)
    assert u.shape == (heads, nb, nb)
    idx = np.full((heads, nb, nb), -1, dtype=np.int32)
    cnt = np.empty((heads, nb), dtype=np.int32)
    lw = np.zeros((heads, nb, nb), dtype=np.float64)
    _check(_load().orc_sip_lists(_ptr(q), _ptr(k), _ptr(u), T, H, W, heads, d, block, float(m),
                                 float(pi_scale), nb, _ptr(idx), _ptr(cnt), _ptr(lw)), "sip_lists")
    return idx, cnt, lw
