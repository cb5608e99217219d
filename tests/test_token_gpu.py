"""GPU parity of the token-level radius policy (the warm-up entropy probe, the
voting mask and the attention over the voted lists) against the fp64 oracle,
through the C ABI."""
import math

import numpy as np
import pytest

import oracle
import tra_inputs as ti

torch = pytest.importorskip("torch")
import content_adaptive_sparse_amd as tra  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
L1_REL = 1e-3
ENT_ABS = 2e-4       # fp32 accumulation of the row statistics over N keys
R2_EPS = 1e-5        # the squared radius is formed in fp32


def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def gpu_token_probe(q, k, shape, tau, gamma):
    heads, T, H, W, d = shape
    ent = torch.full((heads, T, H, W), float("nan"), dtype=torch.float32, device="cuda")
    r0 = torch.full((heads, T, H, W), float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_token_probe(dev16(q), dev16(k), T, H, W, heads, d, 64, tau, gamma, ent, r0)
    torch.cuda.synchronize()
    return ent.cpu().numpy(), r0.cpu().numpy()


def gpu_token_mask(r0, shape, gamma, min_votes):
    heads, T, H, W, d = shape
    nb = tra.tra_grid(T, H, W)[2]
    idx = torch.full((heads, nb, nb), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    tra.tra_token_mask(torch.from_numpy(np.ascontiguousarray(r0)).cuda(), T, H, W, heads, 64,
                       gamma, min_votes, idx, cnt)
    torch.cuda.synchronize()
    return idx, cnt


def assert_close(got, ref, what):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    max_abs, l1 = float(err.max()), float(err.sum() / np.abs(ref).sum())
    print(f"[parity] {what}: max_abs={max_abs:.3e} l1_rel={l1:.3e}", flush=True)
    assert np.isfinite(got).all() and max_abs <= MAX_ABS and l1 <= L1_REL, what


def check_entropy(ent_g, r0_g, ent_ref, tau, gamma, what):
    d_ent = np.abs(ent_g.astype(np.float64) - ent_ref)
    # the radius follows the GPU's own entropy through the budget formula
    r0_own = oracle.token_radius(ent_g.astype(np.float64), tau, gamma)
    rel = np.abs(r0_g - r0_own) / r0_own
    print(f"[parity] {what}: entropy max|d|={d_ent.max():.2e}, r0 rel={rel.max():.2e}", flush=True)
    assert d_ent.max() <= ENT_ABS, what
    assert rel.max() <= 2e-6, what


def check_votes(idx_g, cnt_g, r0_g, gamma, min_votes, rows, what):
    """GPU lists of the given (head * nb + block) rows lie between the oracle's
    lists for the squared radius scaled by 1 - eps and 1 + eps."""
    heads, T, H, W = r0_g.shape
    nb = tra.tra_grid(T, H, W)[2]
    r0 = r0_g.astype(np.float64)
    lo_i, lo_c = oracle.token_lists(r0, gamma, min_votes, rows=rows, r2_scale=1 - R2_EPS)
    hi_i, hi_c = oracle.token_lists(r0, gamma, min_votes, rows=rows, r2_scale=1 + R2_EPS)
    ex_i, ex_c = oracle.token_lists(r0, gamma, min_votes, rows=rows)
    ig = idx_g.reshape(heads * nb, nb)[rows]
    cg = cnt_g.reshape(-1)[rows]
    differ = 0
    for n in range(len(rows)):
        g_ = ig[n, :cg[n]].tolist()
        assert g_ == sorted(g_), f"{what}: row {rows[n]} not ascending"
        lo, hi = set(lo_i[n, :lo_c[n]]), set(hi_i[n, :hi_c[n]])
        assert lo <= set(g_) <= hi, f"{what}: row {rows[n]} outside the rounding bracket"
        differ += g_ != ex_i[n, :ex_c[n]].tolist()
    print(f"[parity] {what}: {len(rows)} lists, {differ} differ from exact arithmetic "
          f"(within the rounding bracket)", flush=True)
    # fp32 squared radii could flip a decision within rounding of a lattice
    # distance; on these seeded inputs none does
    assert differ == 0, f"{what}: {differ} lists differ from exact arithmetic"


SMALL = [
    # (T, H, W, heads, d, tau, gamma, min_votes)
    (3, 20, 28, 2, 128, 1.0, 0.5, 1),
    (2, 13, 9, 1, 64, 4.0, 0.0, 1),
    (4, 16, 24, 2, 128, 0.3, 1.0, 8),
    (1, 5, 7, 1, 64, 1.0, 0.5, 1),
    (5, 8, 8, 1, 128, 2.0, 0.2, 64),
    (2, 8, 200, 1, 128, 1.0, 0.5, 1),   # one tile row: no pair has its lower block
    (2, 70, 6, 1, 64, 1.0, 0.3, 1),     # one ragged tile column of 9 tiles
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])))
def test_token_policy_small_grids(case):
    T, H, W, heads, d, tau, gamma, mv = case
    shape = (heads, T, H, W, d)
    print(f"[case] token policy {case}", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=T + H, family=41)
    ent_g, r0_g = gpu_token_probe(q, k, shape, tau, gamma)
    check_entropy(ent_g, r0_g, oracle.token_entropy(q, k), tau, gamma, f"token probe {case[:5]}")
    idx, cnt = gpu_token_mask(r0_g, shape, gamma, mv)
    nb = tra.tra_grid(T, H, W)[2]
    check_votes(idx.cpu().numpy(), cnt.cpu().numpy(), r0_g, gamma, mv, np.arange(heads * nb),
                f"token mask {case[:5]}")
    # the whole path in one call equals the staged calls, and the oracle's
    # attention over the same lists
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    tra.tra_token_attention(qd, kd, vd, T, H, W, heads, d, 64, tau, gamma, mv, out)
    staged = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn(qd, kd, vd, T, H, W, heads, d, 64, idx, cnt, nb, staged)
    torch.cuda.synchronize()
    assert torch.equal(out, staged)
    rows = np.arange(heads * T * H * W)
    ref = oracle.attention_lists_rows(q, k, v, idx.cpu().numpy(), cnt.cpu().numpy(), rows)
    assert_close(out.cpu().numpy().reshape(-1, d), ref, f"token attention {case[:5]}")


@pytest.mark.parametrize("mixed", [False, True], ids=["negative", "mixed"])
def test_token_entropy_negative_logit_rows(mixed):
    # Rows whose every logit is far below zero (and, mixed, rows of both signs
    # side by side) on ragged grids: a padded key must never stand in for a
    # row's max, and the base-2 online state must not lose the row.
    for T, H, W, heads, d in ((3, 20, 28, 2, 128), (2, 13, 9, 1, 64)):
        shape = (heads, T, H, W, d)
        print(f"[case] token entropy, negative logits {shape} mixed={mixed}", flush=True)
        q, k, _ = ti.aligned_qkv(T, H, W, heads, d, seed=17, mixed_signs=mixed)
        ent_g, r0_g = gpu_token_probe(q, k, shape, 1.0, 0.5)
        check_entropy(ent_g, r0_g, oracle.token_entropy(q, k), 1.0, 0.5,
                      f"token probe, negative logits {shape}")


def test_token_policy_wan_layer_sampled():
    c = ti.WORKLOADS[ti.WAN13B_81F]
    shape = (c.heads, c.T, c.H, c.W, c.d)
    tau, gamma, mv = 1.0, 0.5, 1
    print(f"[case] token policy {c.name}", flush=True)
    q, k, v = ti.make_workload_inputs(ti.WAN13B_81F)
    ent_g, r0_g = gpu_token_probe(q, k, shape, tau, gamma)
    N = c.T * c.H * c.W
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(c.heads * N, size=200, replace=False))
    ref = oracle.token_entropy_rows(q, k, rows)
    got = ent_g.reshape(-1)[rows]
    print(f"[parity] Wan layer entropy ({rows.size} rows): max|d|={np.abs(got - ref).max():.2e}, "
          f"H in [{ref.min():.2f}, {ref.max():.2f}] of ln N = {math.log(N):.2f}", flush=True)
    assert np.abs(got - ref).max() <= ENT_ABS
    idx, cnt = gpu_token_mask(r0_g, shape, gamma, mv)
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    brows = np.sort(rng.choice(c.heads * nb, size=60, replace=False))
    check_votes(idx.cpu().numpy(), cnt.cpu().numpy(), r0_g, gamma, mv, brows, "Wan layer token mask")
    density = cnt.cpu().numpy().sum() / (c.heads * nb * nb)
    print(f"[parity] Wan layer token lists: density {density:.4f}", flush=True)
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_token_attention(dev16(q), dev16(k), dev16(v), c.T, c.H, c.W, c.heads, c.d, 64, tau,
                            gamma, mv, out)
    torch.cuda.synchronize()
    qrows = np.sort(rng.choice(c.heads * N, size=400, replace=False))
    ref = oracle.attention_lists_rows(q, k, v, idx.cpu().numpy(), cnt.cpu().numpy(), qrows)
    assert_close(out.cpu().numpy().reshape(-1, c.d)[qrows], ref, "Wan layer token attention")


def gpu_token_warmup(q, k, v, shape, tau, gamma):
    heads, T, H, W, d = shape
    out = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    ent = torch.full((heads, T, H, W), float("nan"), dtype=torch.float32, device="cuda")
    r0 = torch.full((heads, T, H, W), float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_token_warmup(dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64, tau, gamma, out,
                         ent, r0)
    torch.cuda.synchronize()
    return out, ent.cpu().numpy(), r0.cpu().numpy()


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:5])))
def test_fused_warmup_small_grids(case):
    # The warm-up fused into dense attention: the output is the dense attention
    # (bit-equal to tra_attn's dense mode), and every token's entropy and base
    # radius match the oracle (and the radius follows the GPU's own entropy).
    T, H, W, heads, d, tau, gamma, _ = case
    shape = (heads, T, H, W, d)
    print(f"[case] fused warm-up {case}", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=T + W, family=42)
    out, ent_g, r0_g = gpu_token_warmup(q, k, v, shape, tau, gamma)
    check_entropy(ent_g, r0_g, oracle.token_entropy(q, k), tau, gamma, f"fused warm-up {case[:5]}")
    dense = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn(dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64, None, None, 0, dense)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    nb = tra.tra_grid(T, H, W)[2]
    ref = oracle.attention(q, k, v, oracle.dense_radii(heads, nb))
    assert_close(out.cpu().numpy(), ref, f"fused warm-up output {case[:5]}")


@pytest.mark.parametrize("mixed", [False, True], ids=["negative", "mixed"])
def test_fused_warmup_negative_logit_rows(mixed):
    for T, H, W, heads, d in ((3, 20, 28, 2, 128), (2, 13, 9, 1, 64)):
        shape = (heads, T, H, W, d)
        print(f"[case] fused warm-up, negative logits {shape} mixed={mixed}", flush=True)
        q, k, v = ti.aligned_qkv(T, H, W, heads, d, seed=19, mixed_signs=mixed)
        out, ent_g, r0_g = gpu_token_warmup(q, k, v, shape, 1.0, 0.5)
        check_entropy(ent_g, r0_g, oracle.token_entropy(q, k), 1.0, 0.5,
                      f"fused warm-up, negative logits {shape}")
        nb = tra.tra_grid(T, H, W)[2]
        ref = oracle.attention(q, k, v, oracle.dense_radii(heads, nb))
        assert_close(out.cpu().numpy(), ref, f"fused warm-up output, negative logits {shape}")


def test_fused_warmup_wan_layer():
    # The Wan2.1-1.3B 81-frame layer: entropy of one random token of every query
    # block (and 200 more) against the oracle; the voting lists of the fused
    # radii within the rounding bracket; the output on sampled rows.
    c = ti.WORKLOADS[ti.WAN13B_81F]
    shape = (c.heads, c.T, c.H, c.W, c.d)
    tau, gamma, mv = 1.0, 0.5, 1
    print(f"[case] fused warm-up {c.name}", flush=True)
    q, k, v = ti.make_workload_inputs(ti.WAN13B_81F)
    out, ent_g, r0_g = gpu_token_warmup(q, k, v, shape, tau, gamma)
    N = c.T * c.H * c.W
    nby, nbx = -(-c.H // 8), -(-c.W // 8)
    rng = np.random.default_rng(9)
    rows = []
    for h in range(c.heads):
        for t in range(c.T):
            for by in range(nby):
                for bx in range(nbx):
                    y = 8 * by + int(rng.integers(0, min(8, c.H - 8 * by)))
                    x = 8 * bx + int(rng.integers(0, min(8, c.W - 8 * bx)))
                    rows.append(h * N + (t * c.H + y) * c.W + x)
    rows = np.union1d(np.array(rows), rng.choice(c.heads * N, size=200, replace=False))
    ref = oracle.token_entropy_rows(q, k, rows)
    got = ent_g.reshape(-1)[rows]
    print(f"[parity] fused warm-up entropy ({rows.size} rows): max|d|={np.abs(got - ref).max():.2e}",
          flush=True)
    assert np.abs(got - ref).max() <= ENT_ABS
    r0_own = oracle.token_radius(ent_g.astype(np.float64), tau, gamma)
    assert (np.abs(r0_g - r0_own) / r0_own).max() <= 2e-6
    idx, cnt = gpu_token_mask(r0_g, shape, gamma, mv)
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    brows = np.sort(rng.choice(c.heads * nb, size=60, replace=False))
    check_votes(idx.cpu().numpy(), cnt.cpu().numpy(), r0_g, gamma, mv, brows,
                "fused warm-up token mask")
    qrows = np.sort(rng.choice(c.heads * N, size=400, replace=False))
    ref = oracle.attention_rows(q, k, v, oracle.dense_radii(c.heads, nb), qrows)
    assert_close(out.cpu().numpy().reshape(-1, c.d)[qrows], ref, "fused warm-up output")
