"""GPU parity of sampling with inclusion-probability weighting: the sampled
lists and their log-weights, and the weighted block-sparse attention, against
the fp64 oracle through the C ABI (caller-supplied uniforms on both sides)."""
import numpy as np
import pytest

import oracle
import tra_inputs as ti

torch = pytest.importorskip("torch")
import content_adaptive_sparse_amd as tra  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
L1_REL = 1e-3
PI_EPS = 1e-5   # inclusion probabilities are formed in fp32


def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def assert_close(got, ref, what):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    max_abs, l1 = float(err.max()), float(err.sum() / np.abs(ref).sum())
    print(f"[parity] {what}: max_abs={max_abs:.3e} l1_rel={l1:.3e}", flush=True)
    assert np.isfinite(got).all() and max_abs <= MAX_ABS and l1 <= L1_REL, what


def gpu_sip(q, k, u, shape, m):
    heads, T, H, W, d = shape
    nb = tra.tra_grid(T, H, W)[2]
    idx = torch.full((heads, nb, nb), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    lw = torch.full((heads, nb, nb), float("nan"), dtype=torch.float32, device="cuda")
    ud = torch.from_numpy(u.astype(np.float32)).cuda()
    tra.tra_sip_mask(dev16(q), dev16(k), ud, T, H, W, heads, d, 64, m, idx, cnt, lw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), lw.cpu().numpy()


def check_sip(q, k, u, m, idx_g, cnt_g, lw_g, what):
    """GPU lists lie between the oracle's at pi (1 -+ eps); common entries'
    log-weights agree."""
    heads, nb, _ = idx_g.shape
    u64 = u.astype(np.float32).astype(np.float64)  # the values the GPU compared
    lo_i, lo_c, _ = oracle.sip_lists(q, k, u64, m, pi_scale=1 - PI_EPS)
    hi_i, hi_c, _ = oracle.sip_lists(q, k, u64, m, pi_scale=1 + PI_EPS)
    ex_i, ex_c, ex_w = oracle.sip_lists(q, k, u64, m)
    differ, wmax = 0, 0.0
    for h in range(heads):
        for b in range(nb):
            g_ = idx_g[h, b, :cnt_g[h, b]].tolist()
            assert g_ == sorted(g_) and b in g_, f"{what}: row {h},{b}"
            lo, hi = set(lo_i[h, b, :lo_c[h, b]]), set(hi_i[h, b, :hi_c[h, b]])
            assert lo <= set(g_) <= hi, f"{what}: row {h},{b} outside the rounding bracket"
            ex = dict(zip(ex_i[h, b, :ex_c[h, b]].tolist(), ex_w[h, b, :ex_c[h, b]].tolist()))
            differ += g_ != sorted(ex)
            for kb, w in zip(g_, lw_g[h, b, :cnt_g[h, b]].tolist()):
                if kb in ex:
                    wmax = max(wmax, abs(w - ex[kb]))
    print(f"[parity] {what}: {heads * nb} lists, {differ} differ from exact arithmetic, "
          f"log-weight max|d|={wmax:.2e}", flush=True)
    assert wmax <= 1e-4, what
    # fp32 inclusion probabilities could flip a draw within rounding of pi; on
    # these seeded inputs and uniforms none does
    assert differ == 0, f"{what}: {differ} lists differ from exact arithmetic"


SMALL = [
    # (T, H, W, heads, d, m)
    (3, 20, 28, 2, 128, 3.0),
    (2, 13, 9, 1, 64, 1.5),
    (4, 16, 24, 2, 128, 0.5),
    (5, 8, 8, 1, 128, 1e9),
    (2, 8, 200, 1, 128, 4.0),   # one tile row: no pair has its lower block
    (2, 70, 6, 2, 64, 2.0),     # one ragged tile column of 9 tiles
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])))
def test_sip_small_grids(case):
    T, H, W, heads, d, m = case
    shape = (heads, T, H, W, d)
    print(f"[case] sip {case}", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=T * 7 + W, family=51)
    nb = tra.tra_grid(T, H, W)[2]
    u = np.random.default_rng(T + H).random((heads, nb, nb))
    idx, cnt, lw = gpu_sip(q, k, u, shape, m)
    check_sip(q, k, u, m, idx, cnt, lw, f"sip lists {case[:5]}")
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn_weighted(dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64,
                          torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                          torch.from_numpy(lw).cuda(), nb, out)
    torch.cuda.synchronize()
    rows = np.arange(heads * T * H * W)
    ref = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=lw.astype(np.float64))
    assert_close(out.cpu().numpy().reshape(-1, d), ref, f"sip attention {case[:5]}")


@pytest.mark.parametrize("mixed", [False, True], ids=["negative", "mixed"])
def test_sip_negative_logit_rows(mixed):
    # Sampling and weighted attention where every logit of a row is far below
    # zero (or rows of both signs side by side), on a ragged grid.
    T, H, W, heads, d, m = 3, 20, 28, 2, 128, 3.0
    shape = (heads, T, H, W, d)
    print(f"[case] sip, negative logits {shape} mixed={mixed}", flush=True)
    q, k, v = ti.aligned_qkv(T, H, W, heads, d, seed=19, mixed_signs=mixed)
    nb = tra.tra_grid(T, H, W)[2]
    u = np.random.default_rng(5).random((heads, nb, nb))
    idx, cnt, lw = gpu_sip(q, k, u, shape, m)
    check_sip(q, k, u, m, idx, cnt, lw, f"sip lists, negative logits {shape}")
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn_weighted(dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64,
                          torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                          torch.from_numpy(lw).cuda(), nb, out)
    torch.cuda.synchronize()
    rows = np.arange(heads * T * H * W)
    ref = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=lw.astype(np.float64))
    assert_close(out.cpu().numpy().reshape(-1, d), ref, f"sip attention, negative logits {shape}")


def test_weighted_attention_with_zero_weights_is_tra_attn():
    T, H, W, heads, d = 3, 24, 40, 2, 128
    shape = (heads, T, H, W, d)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=12, family=52)
    nb = tra.tra_grid(T, H, W)[2]
    u = np.random.default_rng(9).random((heads, nb, nb))
    idx, cnt, _ = gpu_sip(q, k, u, shape, 4.0)
    args = (dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64)
    a = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ic, cc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    tra.tra_attn_weighted(*args, ic, cc, torch.zeros(heads, nb, nb, device="cuda"), nb, a)
    tra.tra_attn(*args, ic, cc, nb, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 128])
def test_weighted_walk_cases(d):
    # Weighted walks of caller lists on a grid with edge tiles (20 rows: the
    # last tile row holds 4 real rows; 44 columns: 4 real columns in the last
    # tile column): empty lists (zeros), duplicates (each occurrence counts
    # with its own weight), entries outside [0, nb) skipped, counts beyond
    # maxcnt clamped, descending and shuffled lists, lists longer than one and
    # two 64-entry windows, weights of both signs.  Every output row against
    # the fp64 oracle.
    T, H, W, heads = 3, 20, 44, 2
    shape = (heads, T, H, W, d)
    print(f"[case] weighted walks {shape}", flush=True)
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=31)
    nb = tra.tra_grid(T, H, W)[2]
    maxcnt = 150
    rng = np.random.default_rng(32)
    idx = np.full((heads, nb, maxcnt), -1, dtype=np.int32)
    cnt = np.zeros((heads, nb), dtype=np.int32)
    lw = np.zeros((heads, nb, maxcnt), dtype=np.float32)
    for h in range(heads):
        for b in range(nb):
            kind = (h * nb + b) % 7
            if kind == 0:
                continue  # empty list
            if kind == 1:  # ascending, unique
                row = np.sort(rng.choice(nb, size=rng.integers(1, nb + 1), replace=False))
            elif kind == 2:  # descending
                row = np.sort(rng.choice(nb, size=rng.integers(1, nb + 1), replace=False))[::-1]
            elif kind == 3:  # duplicates, shuffled, past two windows
                row = rng.integers(0, nb, size=rng.integers(129, maxcnt + 1))
            elif kind == 4:  # entries outside [0, nb) among valid ones
                row = rng.integers(-4, nb + 4, size=rng.integers(2, 80))
                row[0] = b
            elif kind == 5:  # count beyond maxcnt: clamped
                row = rng.integers(0, nb, size=maxcnt)
                cnt[h, b] = maxcnt + 17
            else:  # own block only
                row = np.array([b])
            idx[h, b, :len(row)] = row
            cnt[h, b] = max(cnt[h, b], len(row))
            lw[h, b, :len(row)] = rng.uniform(-1.0, 3.0, size=len(row))
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn_weighted(dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64,
                          torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                          torch.from_numpy(lw).cuda(), maxcnt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(-1, d)
    rows = np.arange(heads * T * H * W)
    ref = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=lw.astype(np.float64))
    assert_close(got, ref, f"weighted walks d={d}")
    empty = np.abs(ref).sum(axis=1) == 0
    assert empty.any() and (got[empty] == 0).all()


def test_sip_wan_layer_sampled():
    c = ti.WORKLOADS[ti.WAN13B_81F]
    shape = (c.heads, c.T, c.H, c.W, c.d)
    m = 64.0
    print(f"[case] sip {c.name}, m = {m}", flush=True)
    q, k, v = ti.make_workload_inputs(ti.WAN13B_81F)
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    u = np.random.default_rng(3).random((c.heads, nb, nb)).astype(np.float32)
    idx, cnt, lw = gpu_sip(q, k, u, shape, m)
    print(f"[parity] Wan layer sip: density {cnt.sum() / (c.heads * nb * nb):.4f}", flush=True)
    assert (lw[idx >= 0] >= -1e-6).all()  # pi <= 1
    check_sip(q, k, u, m, idx, cnt, lw, "Wan layer sip lists")
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn_weighted(dev16(q), dev16(k), dev16(v), c.T, c.H, c.W, c.heads, c.d, 64,
                          torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                          torch.from_numpy(lw).cuda(), nb, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(c.heads * c.T * c.H * c.W, size=400, replace=False))
    ref = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=lw.astype(np.float64))
    assert_close(out.cpu().numpy().reshape(-1, c.d)[rows], ref, "Wan layer sip attention")
