"""Python binding of the entropy-radius block-sparse attention library (gfx950).

Argument marshalling only: every function forwards to the C ABI of
``libtra_attention.so`` (declared in ``include/tra_attention.h``) with the
same name and argument order.  Tensors are torch tensors on the GPU
(bf16 q/k/v, fp32 out, int32 radius/idx/cnt); torch provides device memory
and the stream, nothing else.  Integers are accepted in place of tensors as raw
device pointers.  There is no fallback: if the HIP library is not built,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

__all__ = [
    "TRA_RADIUS_INF", "TraError", "library", "tra_attention", "tra_probe", "tra_mask",
    "tra_attn", "tra_grid", "tra_maxcnt", "tra_status_string", "tra_version",
    "tra_plan_bytes", "tra_plan", "tra_attn_plan", "tra_token_probe", "tra_token_mask",
    "tra_token_attention", "tra_token_warmup", "tra_sip_mask", "tra_attn_weighted",
    "tra_workspace_bytes", "tra_time_attn", "tra_release_scratch", "tra_probe_static",
    "tra_static_scratch_bytes", "tra_plan_radius", "tra_time_attn_plan",
    "tra_profile_begin", "tra_profile_end", "KERNEL_KINDS",
]

TRA_RADIUS_INF = 2147483647
KERNEL_KINDS = ("pack_pool", "entropy", "mask", "attn", "fill", "order", "walk",
                "token_entropy", "token_mask", "sip", "vmax", "pair")

_lib = None


class TraError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {tra_status_string(status)} ({status})")
        self.status = status


def library() -> ctypes.CDLL:
    """Load ``libtra_attention.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing "
                "(run `python -m content_adaptive_sparse_amd.build` or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.tra_status_string.argtypes = [I]
        lib.tra_status_string.restype = ctypes.c_char_p
        lib.tra_version.argtypes = []
        lib.tra_version.restype = I
        lib.tra_grid.argtypes = [I, I, I, I, P, P, P]
        lib.tra_grid.restype = I
        lib.tra_maxcnt.argtypes = [I, I, I, I, I]
        lib.tra_maxcnt.restype = L
        lib.tra_attention.argtypes = [P, P, P, I, I, I, I, I, I, I, I, P, P]
        lib.tra_attention.restype = I
        lib.tra_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        lib.tra_workspace_bytes.restype = L
        lib.tra_probe.argtypes = [P, P, I, I, I, I, I, I, I, I, P, P, P, P]
        lib.tra_probe.restype = I
        lib.tra_probe_static.argtypes = [P, P, I, I, I, I, I, I, I, I, P, P, P]
        lib.tra_probe_static.restype = I
        lib.tra_static_scratch_bytes.argtypes = []
        lib.tra_static_scratch_bytes.restype = L
        lib.tra_mask.argtypes = [P, I, I, I, I, I, I, P, P, P]
        lib.tra_mask.restype = I
        lib.tra_attn.argtypes = [P, P, P, I, I, I, I, I, I, P, P, L, P, P]
        lib.tra_attn.restype = I
        lib.tra_plan_bytes.argtypes = [I, I, I, I, I, L]
        lib.tra_plan_bytes.restype = L
        lib.tra_plan.argtypes = [P, P, L, I, I, I, I, I, P, P]
        lib.tra_plan.restype = I
        lib.tra_attn_plan.argtypes = [P, P, P, I, I, I, I, I, I, P, L, P, P]
        lib.tra_attn_plan.restype = I
        lib.tra_plan_radius.argtypes = [P, I, I, I, I, I, I, P, P]
        lib.tra_plan_radius.restype = I
        F = ctypes.c_float
        lib.tra_token_probe.argtypes = [P, P, I, I, I, I, I, I, F, F, P, P, P]
        lib.tra_token_probe.restype = I
        lib.tra_token_mask.argtypes = [P, I, I, I, I, I, F, I, P, P, P]
        lib.tra_token_mask.restype = I
        lib.tra_token_attention.argtypes = [P, P, P, I, I, I, I, I, I, F, F, I, P, P]
        lib.tra_token_attention.restype = I
        lib.tra_token_warmup.argtypes = [P, P, P, I, I, I, I, I, I, F, F, P, P, P, P]
        lib.tra_token_warmup.restype = I
        lib.tra_time_attn.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, L, I, P,
                                      ctypes.POINTER(F), P]
        lib.tra_time_attn.restype = I
        lib.tra_time_attn_plan.argtypes = [P, P, P, I, I, I, I, I, I, P, L, I, P,
                                           ctypes.POINTER(F), P]
        lib.tra_time_attn_plan.restype = I
        lib.tra_release_scratch.argtypes = []
        lib.tra_release_scratch.restype = I
        lib.tra_sip_mask.argtypes = [P, P, P, I, I, I, I, I, I, F, P, P, P, P]
        lib.tra_sip_mask.restype = I
        lib.tra_attn_weighted.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, L, P, P]
        lib.tra_attn_weighted.restype = I
        lib.tra_profile_begin.argtypes = []
        lib.tra_profile_begin.restype = I
        lib.tra_profile_end.argtypes = [P, P, I]
        lib.tra_profile_end.restype = I
        _lib = lib
    return _lib


def _ptr(x, dtype=None, what="tensor"):
    """Device pointer of a contiguous GPU tensor (or a raw int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and x.dtype not in dtype:
        raise ValueError(f"{what} has dtype {x.dtype}, expected one of {dtype}")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _bf16():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def _f32():
    import torch
    return (torch.float32,)


def _i32():
    import torch
    return (torch.int32,)


def _check(status: int, what: str):
    if status != 0:
        raise TraError(status, what)


def tra_status_string(status: int) -> str:
    return library().tra_status_string(int(status)).decode()


def tra_version() -> int:
    return library().tra_version()


def tra_grid(T: int, H: int, W: int, block: int = 64):
    """(nby, nbx, nb) of the tile grid."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(library().tra_grid(T, H, W, block, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "tra_grid")
    return a.value, b.value, c.value


def tra_maxcnt(T: int, H: int, W: int, block: int, r_max: int) -> int:
    n = library().tra_maxcnt(T, H, W, block, r_max)
    if n < 0:
        raise TraError(int(n), "tra_maxcnt")
    return n


def tra_attention(q, k, v, T, H, W, heads, head_dim, block, r_min, r_max, out, stream=None):
    _check(library().tra_attention(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, r_min, r_max, _ptr(out, _f32(), "out"), _stream(stream)), "tra_attention")


def tra_workspace_bytes(T: int, H: int, W: int, heads: int, head_dim: int, block: int,
                        r_max: int) -> int:
    n = library().tra_workspace_bytes(T, H, W, heads, head_dim, block, r_max)
    if n < 0:
        raise TraError(int(n), "tra_workspace_bytes")
    return n


def tra_probe(q, k, T, H, W, heads, head_dim, block, r_min, r_max, radius, h_norm=None,
              ws=None, stream=None):
    _check(library().tra_probe(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), T, H, W, heads, head_dim, block, r_min,
        r_max, _ptr(radius, _i32(), "radius"), _ptr(h_norm, _f32(), "h_norm"),
        _ptr(ws, None, "ws"), _stream(stream)), "tra_probe")


def tra_probe_static(q, k, T, H, W, heads, head_dim, block, r_min, r_max, radius, h_norm=None,
                     stream=None):
    _check(library().tra_probe_static(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), T, H, W, heads, head_dim, block, r_min,
        r_max, _ptr(radius, _i32(), "radius"), _ptr(h_norm, _f32(), "h_norm"), _stream(stream)),
        "tra_probe_static")


def tra_static_scratch_bytes() -> int:
    return int(library().tra_static_scratch_bytes())


def tra_mask(radius, T, H, W, heads, block, r_max, idx, cnt, stream=None):
    _check(library().tra_mask(
        _ptr(radius, _i32(), "radius"), T, H, W, heads, block, r_max, _ptr(idx, _i32(), "idx"),
        _ptr(cnt, _i32(), "cnt"), _stream(stream)), "tra_mask")


def tra_attn(q, k, v, T, H, W, heads, head_dim, block, idx, cnt, maxcnt, out, stream=None):
    _check(library().tra_attn(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, _ptr(idx, _i32(), "idx"), _ptr(cnt, _i32(), "cnt"), int(maxcnt),
        _ptr(out, _f32(), "out"), _stream(stream)), "tra_attn")


def tra_plan_bytes(T: int, H: int, W: int, heads: int, block: int, maxcnt: int) -> int:
    n = library().tra_plan_bytes(T, H, W, heads, block, int(maxcnt))
    if n < 0:
        raise TraError(int(n), "tra_plan_bytes")
    return n


def tra_plan(idx, cnt, maxcnt, T, H, W, heads, block, plan, stream=None):
    """Walk plan of the lists into ``plan`` (a GPU uint8 tensor of tra_plan_bytes bytes)."""
    _check(library().tra_plan(
        _ptr(idx, _i32(), "idx"), _ptr(cnt, _i32(), "cnt"), int(maxcnt), T, H, W, heads, block,
        _ptr(plan, None, "plan"), _stream(stream)), "tra_plan")


def tra_plan_radius(radius, T, H, W, heads, block, r_max, plan, stream=None):
    """Walk plan of the radius mask's lists straight from the radii into ``plan``
    (tra_plan_bytes with maxcnt = tra_maxcnt(..., r_max))."""
    _check(library().tra_plan_radius(
        _ptr(radius, _i32(), "radius"), T, H, W, heads, block, int(r_max),
        _ptr(plan, None, "plan"), _stream(stream)), "tra_plan_radius")


def tra_attn_plan(q, k, v, T, H, W, heads, head_dim, block, plan, maxcnt, out, stream=None):
    _check(library().tra_attn_plan(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, _ptr(plan, None, "plan"), int(maxcnt), _ptr(out, _f32(), "out"),
        _stream(stream)), "tra_attn_plan")


def tra_token_probe(q, k, T, H, W, heads, head_dim, block, tau, gamma, entropy, r0,
                    stream=None):
    _check(library().tra_token_probe(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), T, H, W, heads, head_dim, block, float(tau),
        float(gamma), _ptr(entropy, _f32(), "entropy"), _ptr(r0, _f32(), "r0"), _stream(stream)),
        "tra_token_probe")


def tra_token_mask(r0, T, H, W, heads, block, gamma, min_votes, idx, cnt, stream=None):
    _check(library().tra_token_mask(
        _ptr(r0, _f32(), "r0"), T, H, W, heads, block, float(gamma), int(min_votes),
        _ptr(idx, _i32(), "idx"), _ptr(cnt, _i32(), "cnt"), _stream(stream)), "tra_token_mask")


def tra_token_attention(q, k, v, T, H, W, heads, head_dim, block, tau, gamma, min_votes, out,
                        stream=None):
    _check(library().tra_token_attention(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, float(tau), float(gamma), int(min_votes), _ptr(out, _f32(), "out"),
        _stream(stream)), "tra_token_attention")


def tra_token_warmup(q, k, v, T, H, W, heads, head_dim, block, tau, gamma, out, entropy, r0,
                     stream=None):
    _check(library().tra_token_warmup(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, float(tau), float(gamma), _ptr(out, _f32(), "out"),
        _ptr(entropy, _f32(), "entropy"), _ptr(r0, _f32(), "r0"), _stream(stream)),
        "tra_token_warmup")


def tra_time_attn(q, k, v, T, H, W, heads, head_dim, block, idx, cnt, lw, maxcnt, reps, out,
                  stream=None) -> float:
    """Mean milliseconds of one attention-kernel launch over ``reps`` back-to-back
    launches (lists as for tra_attn_weighted; idx = cnt = None is the dense mode)."""
    ms = ctypes.c_float()
    _check(library().tra_time_attn(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, _ptr(idx, _i32(), "idx"), _ptr(cnt, _i32(), "cnt"),
        _ptr(lw, _f32(), "lw"), int(maxcnt), int(reps), _ptr(out, _f32(), "out"),
        ctypes.byref(ms), _stream(stream)), "tra_time_attn")
    return ms.value


def tra_time_attn_plan(q, k, v, T, H, W, heads, head_dim, block, plan, maxcnt, reps, out,
                       stream=None) -> float:
    """Mean milliseconds of one attention-kernel launch along a stored plan
    (plan = None is the dense mode)."""
    ms = ctypes.c_float()
    _check(library().tra_time_attn_plan(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, _ptr(plan, None, "plan"), int(maxcnt), int(reps),
        _ptr(out, _f32(), "out"), ctypes.byref(ms), _stream(stream)), "tra_time_attn_plan")
    return ms.value


def tra_release_scratch():
    _check(library().tra_release_scratch(), "tra_release_scratch")


def tra_sip_mask(q, k, u, T, H, W, heads, head_dim, block, m, idx, cnt, lw, stream=None):
    _check(library().tra_sip_mask(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(u, _f32(), "u"), T, H, W, heads,
        head_dim, block, float(m), _ptr(idx, _i32(), "idx"), _ptr(cnt, _i32(), "cnt"),
        _ptr(lw, _f32(), "lw"), _stream(stream)), "tra_sip_mask")


def tra_attn_weighted(q, k, v, T, H, W, heads, head_dim, block, idx, cnt, lw, maxcnt, out,
                      stream=None):
    _check(library().tra_attn_weighted(
        _ptr(q, _bf16(), "q"), _ptr(k, _bf16(), "k"), _ptr(v, _bf16(), "v"), T, H, W, heads,
        head_dim, block, _ptr(idx, _i32(), "idx"), _ptr(cnt, _i32(), "cnt"),
        _ptr(lw, _f32(), "lw"), int(maxcnt), _ptr(out, _f32(), "out"), _stream(stream)),
        "tra_attn_weighted")


def tra_profile_begin():
    _check(library().tra_profile_begin(), "tra_profile_begin")


def tra_profile_end():
    """Per-kernel-kind (milliseconds, launches) recorded since tra_profile_begin."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    _check(library().tra_profile_end(ms, cnt, n), "tra_profile_end")
    return {name: (ms[i], cnt[i]) for i, name in enumerate(KERNEL_KINDS)}
