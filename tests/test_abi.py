"""The C-ABI library loads, exports what its header declares, and validates
arguments on the host (no GPU needed: every call here returns before any HIP
work is enqueued)."""
import ctypes
import os
import re

import pytest

import content_adaptive_sparse_amd as tra
from content_adaptive_sparse_amd import build as tra_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tra_attention.h")

INF = tra.TRA_RADIUS_INF
OK, EINVAL, EUNSUP = 0, -1, -2
FAKE = 0x1000  # never dereferenced: validation fails before any launch


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tra_build.LIB_PATH):
        tra_build.build()
    return tra.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tra_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ["tra_attention", "tra_probe", "tra_mask", "tra_attn", "tra_maxcnt", "tra_grid",
              "tra_status_string", "tra_version", "tra_profile_begin", "tra_profile_end",
              "tra_plan_bytes", "tra_plan", "tra_attn_plan", "tra_plan_radius",
              "tra_time_attn_plan"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_status_strings(lib):
    assert tra.tra_status_string(0) == "TRA_OK"
    assert tra.tra_status_string(-1) == "TRA_ERR_INVALID_ARG"
    assert tra.tra_status_string(-2) == "TRA_ERR_UNSUPPORTED"
    assert tra.tra_status_string(-3) == "TRA_ERR_HIP"
    assert tra.tra_status_string(-4) == "TRA_ERR_NOMEM"
    assert tra.tra_status_string(-5) == "TRA_ERR_TOO_LARGE"
    assert tra.tra_status_string(7) == "TRA_ERR_UNKNOWN"
    assert tra.tra_version() >= 100


def test_grid_and_maxcnt_closed_forms(lib):
    assert tra.tra_grid(21, 30, 52) == (4, 7, 588)
    assert tra.tra_grid(8, 8, 8) == (1, 1, 8)
    assert tra.tra_grid(33, 45, 80) == (6, 10, 1980)
    assert tra.tra_maxcnt(8, 8, 8, 64, 3) == 7
    assert tra.tra_maxcnt(21, 30, 52, 64, 8) == 476
    assert tra.tra_maxcnt(61, 30, 52, 64, 12) == 700
    assert tra.tra_maxcnt(21, 45, 80, 64, 10) == 1260
    assert tra.tra_maxcnt(33, 45, 80, 64, 16) == 1980
    assert tra.tra_maxcnt(21, 30, 52, 64, INF) == 588
    assert tra.tra_maxcnt(21, 30, 52, 64, 0) == 1
    with pytest.raises(tra.TraError):
        tra.tra_maxcnt(21, 30, 52, 64, -1)
    with pytest.raises(tra.TraError):
        tra.tra_grid(21, 30, 52, 32)


def _attention(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, T=4, H=16, W=16, heads=2, d=128, block=64, r_min=1,
             r_max=4, out=FAKE)
    a.update(kw)
    return lib.tra_attention(a["q"], a["k"], a["v"], a["T"], a["H"], a["W"], a["heads"], a["d"],
                             a["block"], a["r_min"], a["r_max"], a["out"], None)


def test_tra_attention_argument_errors(lib):
    assert _attention(lib, q=None) == EINVAL
    assert _attention(lib, out=None) == EINVAL
    assert _attention(lib, T=0) == EINVAL
    assert _attention(lib, H=-3) == EINVAL
    assert _attention(lib, heads=0) == EINVAL
    assert _attention(lib, r_min=5, r_max=4) == EINVAL
    assert _attention(lib, r_min=-1) == EINVAL
    assert _attention(lib, r_min=INF, r_max=4) == EINVAL
    assert _attention(lib, block=32) == EUNSUP
    assert _attention(lib, d=96) == EUNSUP
    assert _attention(lib, d=256) == EUNSUP
    assert _attention(lib, heads=70000) == EUNSUP
    assert _attention(lib, T=50000, H=50000, W=50000) == EUNSUP


def test_staged_entry_point_argument_errors(lib):
    assert lib.tra_probe(FAKE, FAKE, 4, 16, 16, 2, 128, 64, 1, 4, None, None, None, None) == EINVAL
    assert lib.tra_probe(FAKE, FAKE, 4, 16, 16, 2, 128, 64, 4, 1, FAKE, None, FAKE, None) == EINVAL
    assert lib.tra_probe(FAKE, FAKE, 4, 16, 16, 2, 80, 64, 1, 4, FAKE, None, FAKE, None) == EUNSUP
    assert lib.tra_probe(None, FAKE, 4, 16, 16, 2, 128, 64, 1, 4, FAKE, None, FAKE, None) == EINVAL
    assert lib.tra_mask(FAKE, 4, 16, 16, 2, 64, -1, FAKE, FAKE, None) == EINVAL
    assert lib.tra_mask(None, 4, 16, 16, 2, 64, 3, FAKE, FAKE, None) == EINVAL
    assert lib.tra_mask(FAKE, 4, 16, 16, 2, 16, 3, FAKE, FAKE, None) == EUNSUP
    # idx and cnt must both be given or both be NULL
    assert lib.tra_attn(FAKE, FAKE, FAKE, 4, 16, 16, 2, 128, 64, FAKE, None, 5, FAKE, None) == EINVAL
    assert lib.tra_attn(FAKE, FAKE, FAKE, 4, 16, 16, 2, 128, 64, FAKE, FAKE, 0, FAKE, None) == EINVAL
    assert lib.tra_attn(FAKE, FAKE, FAKE, 4, 16, 16, 2, 64, 64, None, None, 0, None, None) == EINVAL


def test_workspace_bytes_closed_form(lib):
    # tra_probe's workspace: the fp32 block means of q and k, each 256-byte aligned
    def up(x):
        return (x + 255) // 256 * 256

    for (T, H, W, heads, d, r_max) in [(21, 30, 52, 12, 128, 8), (8, 8, 8, 1, 64, 3),
                                       (33, 45, 80, 24, 128, 16), (1, 1, 1, 3, 64, INF)]:
        nb = tra.tra_grid(T, H, W)[2]
        assert tra.tra_workspace_bytes(T, H, W, heads, d, 64, r_max) == 2 * up(heads * nb * d * 4)
    assert lib.tra_workspace_bytes(4, 16, 16, 2, 128, 64, -1) == EINVAL
    assert lib.tra_workspace_bytes(0, 16, 16, 2, 128, 64, 3) == EINVAL
    assert lib.tra_workspace_bytes(4, 16, 16, 2, 96, 64, 3) == EUNSUP
    assert lib.tra_workspace_bytes(4, 16, 16, 2, 128, 32, 3) == EUNSUP


def test_warmup_and_timing_argument_errors(lib):
    F = ctypes.c_float
    ms = F()
    args = (FAKE, FAKE, FAKE, 4, 16, 16, 2, 128, 64)
    # tra_token_warmup: r0 and out required; tau > 0, gamma >= 0
    assert lib.tra_token_warmup(*args, F(1.0), F(0.5), FAKE, None, None, None) == EINVAL
    assert lib.tra_token_warmup(*args, F(1.0), F(0.5), None, None, FAKE, None) == EINVAL
    assert lib.tra_token_warmup(*args, F(0.0), F(0.5), FAKE, None, FAKE, None) == EINVAL
    assert lib.tra_token_warmup(*args, F(1.0), F(-1.0), FAKE, None, FAKE, None) == EINVAL
    assert lib.tra_token_warmup(FAKE, FAKE, FAKE, 4, 16, 16, 2, 96, 64, F(1.0), F(0.5), FAKE,
                                None, FAKE, None) == EUNSUP
    # tra_time_attn: reps in [1, 4096], ms given, idx/cnt together, weights only with lists
    assert lib.tra_time_attn(*args, None, None, None, 0, 0, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn(*args, None, None, None, 0, 4097, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn(*args, None, None, None, 0, 3, FAKE, None, None) == EINVAL
    assert lib.tra_time_attn(*args, FAKE, None, None, 5, 3, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn(*args, None, None, FAKE, 0, 3, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn(*args, FAKE, FAKE, None, 0, 3, FAKE, ctypes.byref(ms), None) == EINVAL


def test_static_probe_argument_errors(lib):
    # validated on the host before the static array is touched
    assert lib.tra_static_scratch_bytes() == 64 << 20
    assert lib.tra_probe_static(FAKE, FAKE, 4, 16, 16, 2, 128, 64, 1, 4, None, None, None) == EINVAL
    assert lib.tra_probe_static(FAKE, FAKE, 4, 16, 16, 2, 80, 64, 1, 4, FAKE, None, None) == EUNSUP
    assert lib.tra_probe_static(FAKE, FAKE, 4, 16, 16, 2, 128, 64, 4, 1, FAKE, None, None) == EINVAL
    # block means of 64 heads of a 33 x 45 x 80 grid need more than the 64 MiB array
    assert lib.tra_probe_static(FAKE, FAKE, 33, 45, 80, 64, 128, 64, 1, 4, FAKE, None, None) == -5


def test_plan_bytes_closed_form(lib):
    def up(x):
        return (x + 255) // 256 * 256

    for (T, H, W, heads, maxcnt) in [(21, 30, 52, 12, 476), (8, 8, 8, 1, 7), (3, 20, 28, 2, 1)]:
        nby, nbx = -(-H // 8), -(-W // 8)
        # item slots per head: vertical pairs or temporal pairs, whichever are more
        items = heads * max(T * ((nby + 1) // 2) * nbx, (T + 1) // 2 * nby * nbx)
        slots = -(-items // 8) * 8
        order = 8 * 2 * -(-items // 8) + 8  # eight ranges of at most twice the mean count, their lengths
        stride = -(-(2 * maxcnt) // 64) * 64
        # work order, walk lengths, walks, pair table (two int32 per item slot)
        want = up(4 * order) + up(4 * slots) + up(4 * slots * stride) + up(8 * slots)
        assert tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt) == want


def test_plan_argument_errors(lib):
    assert lib.tra_plan_bytes(4, 16, 16, 2, 64, 0) == EINVAL
    assert lib.tra_plan_bytes(4, 16, 16, 2, 64, (1 << 30) + 1) == EINVAL
    assert lib.tra_plan_bytes(4, 16, 16, 2, 16, 5) == EUNSUP
    assert lib.tra_plan_bytes(21, 30, 52, 12, 64, 1 << 30) == EUNSUP  # > 2^44 bytes
    assert lib.tra_plan(FAKE, FAKE, 5, 4, 16, 16, 2, 64, None, None) == EINVAL
    assert lib.tra_plan(None, FAKE, 5, 4, 16, 16, 2, 64, FAKE, None) == EINVAL
    assert lib.tra_plan(FAKE, FAKE, 0, 4, 16, 16, 2, 64, FAKE, None) == EINVAL
    assert lib.tra_attn_plan(FAKE, FAKE, FAKE, 4, 16, 16, 2, 128, 64, None, 5, FAKE, None) == EINVAL
    assert lib.tra_attn_plan(FAKE, FAKE, FAKE, 4, 16, 16, 2, 80, 64, FAKE, 5, FAKE, None) == EUNSUP
    assert lib.tra_attn_plan(FAKE, FAKE, FAKE, 4, 16, 16, 2, 128, 64, FAKE, 0, FAKE, None) == EINVAL
    # tra_plan_radius: radius and plan required, r_max >= 0, block 64
    assert lib.tra_plan_radius(None, 4, 16, 16, 2, 64, 3, FAKE, None) == EINVAL
    assert lib.tra_plan_radius(FAKE, 4, 16, 16, 2, 64, 3, None, None) == EINVAL
    assert lib.tra_plan_radius(FAKE, 4, 16, 16, 2, 64, -1, FAKE, None) == EINVAL
    assert lib.tra_plan_radius(FAKE, 4, 16, 16, 2, 32, 3, FAKE, None) == EUNSUP
    assert lib.tra_plan_radius(FAKE, 4, 16, 16, 0, 64, 3, FAKE, None) == EINVAL
    # tra_time_attn_plan: reps in [1, 4096], ms given, the plan's maxcnt checked when a plan is given
    F = ctypes.c_float
    ms = F()
    args = (FAKE, FAKE, FAKE, 4, 16, 16, 2, 128, 64)
    assert lib.tra_time_attn_plan(*args, FAKE, 5, 0, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn_plan(*args, FAKE, 5, 4097, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn_plan(*args, FAKE, 5, 3, FAKE, None, None) == EINVAL
    assert lib.tra_time_attn_plan(*args, FAKE, 0, 3, FAKE, ctypes.byref(ms), None) == EINVAL
    assert lib.tra_time_attn_plan(*args, FAKE, 5, 3, None, ctypes.byref(ms), None) == EINVAL


def test_profile_switch_without_launches(lib):
    tra.tra_profile_begin()
    res = tra.tra_profile_end()
    assert all(v == (0.0, 0) for v in res.values())


def test_binding_refuses_host_tensors(lib):
    import torch
    x = torch.zeros(4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tra.tra_attention(x, x, x, 1, 1, 4, 1, 1, 64, 0, 0, torch.zeros(4))
