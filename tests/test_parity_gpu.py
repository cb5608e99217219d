"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Bars (the same for every case):
  * radii: identical, except blocks whose oracle h_norm lies within 1e-4 of a
    quantisation boundary k/(r_max - r_min + 1); those are reported;
  * key-block lists: bit-exact (idx[:cnt] and cnt) given the same radii;
  * outputs: max-abs error <= 1e-2 and L1-relative error sum|o - o_ref| /
    sum|o_ref| <= 1e-3 over real tokens, against the oracle run on the GPU's
    own radii.
Small grids compare every output; the full workload shapes compare sampled
rows (the oracle computes them one by one).
"""
import math

import numpy as np
import pytest

import oracle
import tra_inputs as ti

torch = pytest.importorskip("torch")
import content_adaptive_sparse_amd as tra  # noqa: E402

pytestmark = pytest.mark.gpu

INF = tra.TRA_RADIUS_INF
MAX_ABS = 1e-2
L1_REL = 1e-3
BAND = 1e-4
HN_ABS = 1e-5   # fp32 pooled logits and entropy against fp64


# ---------------------------------------------------------------- helpers --

def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def gpu_probe(qd, kd, shape, r_min, r_max):
    heads, T, H, W, d = shape
    nb = tra.tra_grid(T, H, W)[2]
    r = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    hn = torch.empty(heads, nb, dtype=torch.float32, device="cuda")
    tra.tra_probe(qd, kd, T, H, W, heads, d, 64, r_min, r_max, r, hn)
    torch.cuda.synchronize()
    return hn.cpu().numpy(), r.cpu().numpy()


def gpu_mask(radii, shape, r_max):
    heads, T, H, W, d = shape
    nb = tra.tra_grid(T, H, W)[2]
    maxcnt = tra.tra_maxcnt(T, H, W, 64, r_max)
    rd = torch.from_numpy(np.ascontiguousarray(radii, dtype=np.int32)).cuda()
    idx = torch.full((heads, nb, maxcnt), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    tra.tra_mask(rd, T, H, W, heads, 64, r_max, idx, cnt)
    torch.cuda.synchronize()
    return idx, cnt, maxcnt


def gpu_attn(qd, kd, vd, shape, idx=None, cnt=None, maxcnt=0):
    heads, T, H, W, d = shape
    out = torch.full((heads, T, H, W, d), float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn(qd, kd, vd, T, H, W, heads, d, 64, idx, cnt, maxcnt, out)
    torch.cuda.synchronize()
    return out


def gpu_attention(qd, kd, vd, shape, r_min, r_max):
    heads, T, H, W, d = shape
    out = torch.full((heads, T, H, W, d), float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attention(qd, kd, vd, T, H, W, heads, d, 64, r_min, r_max, out)
    torch.cuda.synchronize()
    return out


def assert_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    max_abs = float(err.max())
    l1 = float(err.sum() / np.abs(ref).sum())
    print(f"[parity] {what}: max_abs={max_abs:.3e} l1_rel={l1:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert max_abs <= MAX_ABS, f"{what}: max-abs {max_abs}"
    assert l1 <= L1_REL, f"{what}: L1-relative {l1}"


def boundary_blocks(hn_ref, r_min, r_max):
    R = r_max - r_min + 1
    ks = np.arange(1, R) / R
    if ks.size == 0:
        return np.zeros(hn_ref.shape, dtype=bool)
    return np.min(np.abs(hn_ref[..., None] - ks), axis=-1) < BAND


def check_radii(hn_gpu, r_gpu, hn_ref, r_ref, r_min, r_max, what):
    R = r_max - r_min + 1
    # the radius follows the stored fp32 h_norm exactly
    own = np.clip(r_min + np.floor(hn_gpu.astype(np.float64) * R), r_min, r_max).astype(np.int64)
    assert np.array_equal(own, r_gpu), f"{what}: radius does not follow its own h_norm"
    band = boundary_blocks(hn_ref, r_min, r_max)
    diff = r_gpu != r_ref
    hn_err = float(np.abs(hn_gpu.astype(np.float64) - hn_ref).max())
    print(f"[parity] {what}: h_norm max|d|={hn_err:.2e}, "
          f"boundary blocks={int(band.sum())}, radius mismatches={int(diff.sum())}", flush=True)
    assert hn_err <= HN_ABS, f"{what}: h_norm max|d| {hn_err}"
    for h, b in zip(*np.nonzero(band)):
        print(f"[boundary] {what} head {h} block {b}: h_norm oracle={hn_ref[h, b]:.7f} "
              f"gpu={hn_gpu[h, b]:.7f} r oracle={r_ref[h, b]} gpu={r_gpu[h, b]}", flush=True)
    assert not (diff & ~band).any(), f"{what}: radius mismatch outside the boundary band"


def check_lists(idx_g, cnt_g, radii, shape, maxcnt, what):
    heads, T, H, W, d = shape
    idx_o, cnt_o = oracle.block_lists(radii, T, H, W, maxcnt=maxcnt)
    cnt_g = cnt_g.cpu().numpy()
    idx_g = idx_g.cpu().numpy()
    assert np.array_equal(cnt_g, cnt_o), f"{what}: cnt differs"
    valid = np.arange(maxcnt)[None, None, :] < cnt_o[..., None]
    assert np.array_equal(np.where(valid, idx_g, -1), np.where(valid, idx_o, -1)), f"{what}: idx differs"


def sample_rows(shape, n, seed=0):
    """Seeded sample of (head * N + token) rows, always including edge-tile tokens."""
    heads, T, H, W, d = shape
    N = T * H * W
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(heads * N, size=min(n, heads * N), replace=False).tolist())
    for h in (0, heads - 1):
        for t, y, x in ((0, 0, 0), (T - 1, H - 1, W - 1), (T // 2, H - 1, 0), (0, 0, W - 1)):
            rows.add(h * N + (t * H + y) * W + x)
    return np.array(sorted(rows), dtype=np.int64)


def item_rows(shape, per_block=1, seed=0):
    """Seeded rows covering every attention work item: for each head and each
    pair of vertically adjacent query blocks (frame t, tile rows 2p and 2p + 1,
    tile column bx), `per_block` random real query tokens of each block of the
    pair (the first drawn among the block's first 32 real queries, the next
    among the rest when there are any, so both waves of a block are reached)."""
    heads, T, H, W, d = shape
    N = T * H * W
    nby, nbx = -(-H // 8), -(-W // 8)
    rng = np.random.default_rng(seed)
    rows = []
    for h in range(heads):
        for t in range(T):
            for by in range(nby):
                for bx in range(nbx):
                    ny, nx = min(8, H - 8 * by), min(8, W - 8 * bx)
                    nq = ny * nx
                    for j in range(per_block):
                        lo, hi = (0, min(32, nq)) if j % 2 == 0 or nq <= 32 else (32, nq)
                        qi = int(rng.integers(lo, hi))
                        y, x = 8 * by + qi // nx, 8 * bx + qi % nx
                        rows.append(h * N + (t * H + y) * W + x)
    return np.unique(np.array(rows, dtype=np.int64))


# ------------------------------------------------------ small full grids --

SMALL = [
    # (T, H, W, heads, d)
    (3, 20, 28, 2, 128),   # 3x4 tiles per frame, ragged bottom and right
    (4, 16, 24, 2, 64),    # exact tiles
    (2, 13, 9, 3, 128),    # 2x2 tiles, heavily ragged
    (1, 5, 7, 1, 64),      # one partial tile: nb = 1
    (1, 1, 1, 2, 128),     # a single token
    (5, 8, 8, 1, 128),     # one tile per frame
    (2, 8, 200, 1, 128),   # one tile row of 25 tiles: no pair has its lower block
    (2, 70, 6, 2, 64),     # one ragged tile column of 9 tiles: the last pair is single
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_grid_staged_path(shape):
    heads, T, H, W, d = shape[3], shape[0], shape[1], shape[2], shape[4]
    shp = (heads, T, H, W, d)
    print(f"[case] staged {shp}", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=1, family=21)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    r_min, r_max = 0, 2
    hn_g, r_g = gpu_probe(qd, kd, shp, r_min, r_max)
    hn_o, r_o = oracle.probe(q, k, r_min, r_max)
    check_radii(hn_g, r_g, hn_o, r_o, r_min, r_max, f"probe {shp}")
    idx, cnt, maxcnt = gpu_mask(r_g, shp, r_max)
    check_lists(idx, cnt, r_g, shp, maxcnt, f"mask {shp}")
    out = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
    ref = oracle.attention(q, k, v, r_g)
    assert_close(out, ref, f"attn {shp}")
    # the fused call gives the same result as the staged calls
    out2 = gpu_attention(qd, kd, vd, shp, r_min, r_max).cpu().numpy()
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("d", [64, 128])
def test_random_radii_and_dense(d):
    T, H, W, heads = 4, 19, 27, 2
    shp = (heads, T, H, W, d)
    print(f"[case] random radii {shp}", flush=True)
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=5, scale=1.5)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    nb = tra.tra_grid(T, H, W)[2]
    rng = np.random.default_rng(3)
    for radii, r_max in ((rng.integers(0, 4, size=(heads, nb)), 3),
                         (np.zeros((heads, nb)), 0),
                         (np.full((heads, nb), 9), 9)):
        radii = radii.astype(np.int32)
        idx, cnt, maxcnt = gpu_mask(radii, shp, r_max)
        check_lists(idx, cnt, radii, shp, maxcnt, f"mask r_max={r_max}")
        out = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
        assert_close(out, oracle.attention(q, k, v, radii), f"attn r_max={r_max} d={d}")
    dense = gpu_attn(qd, kd, vd, shp).cpu().numpy()
    ref = oracle.attention(q, k, v, oracle.dense_radii(heads, nb))
    assert_close(dense, ref, f"dense d={d}")
    dense2 = gpu_attention(qd, kd, vd, shp, INF, INF).cpu().numpy()
    assert np.array_equal(dense, dense2)
    # a radius covering the whole grid keeps every block in the same order: same bits
    idx, cnt, maxcnt = gpu_mask(np.full((heads, nb), 9, dtype=np.int32), shp, 9)
    wide = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
    assert np.array_equal(wide, dense)


def test_tiny_workload_end_to_end():
    c = ti.WORKLOADS[ti.TINY]
    shp = (c.heads, c.T, c.H, c.W, c.d)
    print(f"[case] tiny workload {shp}", flush=True)
    q, k, v = ti.make_workload_inputs(ti.TINY)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    hn_g, r_g = gpu_probe(qd, kd, shp, c.r_min, c.r_max)
    hn_o, r_o = oracle.probe(q, k, c.r_min, c.r_max)
    check_radii(hn_g, r_g, hn_o, r_o, c.r_min, c.r_max, "tiny workload probe")
    out = gpu_attention(qd, kd, vd, shp, c.r_min, c.r_max).cpu().numpy()
    assert_close(out, oracle.attention(q, k, v, r_g), "tiny workload attention")


# --------------------------------------------------------------- edge cases --

def test_list_edge_cases():
    T, H, W, heads, d = 2, 16, 16, 1, 128
    shp = (heads, T, H, W, d)
    print(f"[case] list edge cases {shp}", flush=True)
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=9)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    nb = tra.tra_grid(T, H, W)[2]
    maxcnt = 4
    idx = np.full((heads, nb, maxcnt), -1, dtype=np.int32)
    cnt = np.zeros((heads, nb), dtype=np.int32)
    # block 0: empty list -> zeros; block 1: {1, 5}; block 2: invalid entries
    # are skipped; block 3: cnt beyond maxcnt is clamped; others: own block
    idx[0, 1, :2] = [1, 5]
    cnt[0, 1] = 2
    idx[0, 2, :4] = [2, -3, 99, 6]
    cnt[0, 2] = 4
    idx[0, 3, :4] = [0, 1, 2, 3]
    cnt[0, 3] = 100
    for b in range(4, nb):
        idx[0, b, 0] = b
        cnt[0, b] = 1
    out = gpu_attn(qd, kd, vd, shp, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                   maxcnt).cpu().numpy().reshape(heads, -1, d)
    tok = np.arange(T * H * W).reshape(T, H, W)
    blocks = [tok[t, 8 * by:8 * by + 8, 8 * bx:8 * bx + 8].ravel()
              for t in range(T) for by in range(2) for bx in range(2)]
    qf, kf, vf = (ti.bf16_to_f32(a).astype(np.float64).reshape(heads, -1, d) for a in (q, k, v))

    def ref_rows(qblock, kblocks):
        keys = np.concatenate([blocks[b] for b in kblocks])
        s = qf[0, blocks[qblock]] @ kf[0, keys].T / math.sqrt(d)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        return (w / w.sum(axis=1, keepdims=True)) @ vf[0, keys]

    assert (out[0, blocks[0]] == 0).all()
    assert_close(out[0, blocks[1]], ref_rows(1, [1, 5]), "list {1,5}")
    assert_close(out[0, blocks[2]], ref_rows(2, [2, 6]), "invalid entries skipped")
    assert_close(out[0, blocks[3]], ref_rows(3, [0, 1, 2, 3]), "cnt clamped")
    for b in range(4, nb):
        assert_close(out[0, blocks[b]], ref_rows(b, [b]), f"own block {b}")


def test_list_walk_cases():
    # Each attention work item walks the union of its two query blocks' lists
    # (the plan's pair table): ascending lists merge (overlaps computed once,
    # unions longer than 64 entries), other lists (descending, duplicates)
    # are walked as they stand.  Every block must still see exactly its own
    # list, a duplicate counting twice.
    T, H, W, heads, d = 20, 16, 16, 1, 128
    shp = (heads, T, H, W, d)
    print(f"[case] list walk cases {shp}", flush=True)
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=11)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    nb = tra.tra_grid(T, H, W)[2]
    assert nb == 80
    maxcnt = nb
    lists = {b: [b] for b in range(nb)}
    lists[0] = list(range(nb - 1, -1, -1))          # descending: walked as is
    lists[2] = [5, 5, 7]                            # duplicate counts twice
    lists[1] = list(range(0, nb, 2))                # pair (1, 3): overlapping merge
    lists[3] = list(range(0, nb, 3))
    lists[4] = list(range(nb))                      # pair (4, 6): union of 80 entries
    lists[6] = []
    lists[5] = [nb - 1]                             # pair (5, 7): disjoint
    lists[7] = [0]
    idx = np.full((heads, nb, maxcnt), -1, dtype=np.int32)
    cnt = np.zeros((heads, nb), dtype=np.int32)
    for b, l in lists.items():
        idx[0, b, :len(l)] = l
        cnt[0, b] = len(l)
    out = gpu_attn(qd, kd, vd, shp, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                   maxcnt).cpu().numpy().reshape(heads, -1, d)
    tok = np.arange(T * H * W).reshape(T, H, W)
    blocks = [tok[t, 8 * by:8 * by + 8, 8 * bx:8 * bx + 8].ravel()
              for t in range(T) for by in range(2) for bx in range(2)]
    qf, kf, vf = (ti.bf16_to_f32(a).astype(np.float64).reshape(heads, -1, d) for a in (q, k, v))
    for b in range(nb):
        if not lists[b]:
            assert (out[0, blocks[b]] == 0).all()
            continue
        keys = np.concatenate([blocks[kb] for kb in lists[b]])
        s = qf[0, blocks[b]] @ kf[0, keys].T / math.sqrt(d)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (w / w.sum(axis=1, keepdims=True)) @ vf[0, keys]
        assert_close(out[0, blocks[b]], ref, f"walk block {b} ({len(lists[b])} entries)")


def test_plan_reuse_across_steps():
    # Cross-step reuse: lists decided once (probe + mask on the first step's q, k),
    # turned into a walk plan once, then attention of later steps' q, k, v along
    # the stored plan.  Each step must equal tra_attn with the same lists
    # bit for bit, and the oracle with the same radii within tolerance.
    T, H, W, heads, d = 4, 24, 40, 2, 128
    shp = (heads, T, H, W, d)
    print(f"[case] plan reuse {shp}", flush=True)
    r_min, r_max = 0, 3
    q0, k0, _ = ti.make_inputs(T, H, W, heads, d, seed=3, family=31)
    hn, radii = gpu_probe(dev16(q0), dev16(k0), shp, r_min, r_max)
    idx, cnt, maxcnt = gpu_mask(radii, shp, r_max)
    plan = torch.empty(tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt), dtype=torch.uint8,
                       device="cuda")
    tra.tra_plan(idx, cnt, maxcnt, T, H, W, heads, 64, plan)
    for step in range(2):
        q, k, v = ti.make_inputs(T, H, W, heads, d, seed=40 + step, family=31)
        qd, kd, vd = dev16(q), dev16(k), dev16(v)
        out = torch.full(shp, float("nan"), dtype=torch.float32, device="cuda")
        tra.tra_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan, maxcnt, out)
        ref_gpu = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_gpu), f"step {step}: planned walk differs from tra_attn"
        rows = sample_rows(shp, 600, seed=step)
        ref = oracle.attention_rows(q, k, v, radii, rows)
        assert_close(out.cpu().numpy().reshape(-1, d)[rows], ref, f"plan reuse step {step}")


@pytest.mark.parametrize("case", ["probe", "random", "routing", "wide"])
def test_plan_from_radii(case):
    # The walk plan built straight from radii (tra_plan_radius, the plan
    # tra_attention builds: its own pairing, no lists) gives the same bits as
    # tra_attn on tra_mask's lists of the same radii -- every block meets its own
    # key blocks in ascending order whoever shares its walk.  Random radii include
    # negative values and values above r_max (both clamped like tra_mask clamps
    # them); "routing" is binary routing (radius 1 or TRA_RADIUS_INF); "wide"
    # has more than 256 tiles per frame (the pairing without frame order).
    T, H, W, heads, d = {"routing": (6, 30, 52, 2, 64), "wide": (3, 136, 144, 1, 64)}.get(
        case, (5, 29, 43, 3, 128))
    shp = (heads, T, H, W, d)
    print(f"[case] plan from radii {shp} {case}", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=12, family=36)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    nb = tra.tra_grid(T, H, W)[2]
    rng = np.random.default_rng(21)
    if case == "probe":
        r_max = 4
        _, radii = gpu_probe(qd, kd, shp, 1, r_max)
    elif case in ("random", "wide"):
        r_max = 3
        radii = rng.integers(-2, 6, size=(heads, nb)).astype(np.int32)
    else:
        r_max = INF
        radii = np.where(rng.random((heads, nb)) < 0.2, INF, 1).astype(np.int32)
    idx, cnt, maxcnt = gpu_mask(radii, shp, r_max)
    assert maxcnt == tra.tra_maxcnt(T, H, W, 64, r_max)
    plan = torch.empty(tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt), dtype=torch.uint8,
                       device="cuda")
    tra.tra_plan_radius(torch.from_numpy(radii).cuda(), T, H, W, heads, 64, r_max, plan)
    torch.cuda.synchronize()
    got = plan_pair_table(plan, T, H, W, heads, maxcnt)
    want = radius_pair_table_model(radii, r_max, T, H, W)
    assert np.array_equal(got, want), "pair table differs from the radius rule"
    out = torch.full(shp, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan, maxcnt, out)
    ref_gpu = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_gpu), "walks from radii differ from the lists' walks"
    if case == "probe":
        fused = gpu_attention(qd, kd, vd, shp, 1, r_max)
        assert torch.equal(out, fused), "tra_attention differs from its plan"
    clamped = np.clip(radii, 0, r_max if r_max != INF else None)
    rows = np.union1d(item_rows(shp, 1, seed=3), sample_rows(shp, 0, seed=3))
    ref = oracle.attention_rows(q, k, v, clamped, rows)
    assert_close(out.cpu().numpy().reshape(-1, d)[rows], ref, f"plan from radii ({case})")


def order_class(n):
    """Length class of the work order: the length below 4, else two per octave."""
    n = int(n)
    if n <= 3:
        return n
    e = n.bit_length() - 1
    return 2 * e + ((n >> (e - 1)) & 1)


@pytest.mark.parametrize("case", ["balanced", "capped", "many"])
def test_work_order_ranges(case):
    # The work order deals the walk items to eight XCD ranges: contiguous raster
    # ranges cut at equal shares of the total work (walk length + 4 per item),
    # each of at most cap = 2 ceil(items / 8) items, taken by length class
    # (two per octave, longest first; item order inside a class) into grid
    # slots 8 k + x, -1 past a range's end.  Every item appears once.  The
    # skewed case puts nearly all the work in the first items, so equal-work
    # cuts would leave the later ranges above the cap: the cap moves the cuts.
    # "many" has more than 8192 items (more than eight per thread of the order
    # kernel's workgroup, which then reads the lengths in a loop).
    skewed = case == "capped"
    T, H, W, heads = (21, 45, 80, 16) if case == "many" else (6, 30, 52, 3)
    shp = (heads, T, H, W, 128)
    print(f"[case] work order {shp} {case}", flush=True)
    nb = tra.tra_grid(T, H, W)[2]
    rng = np.random.default_rng(17)
    if skewed:
        radii = np.zeros((heads, nb), dtype=np.int32)
        radii[0, : nb // 4] = 6          # a few long walks at the very start
        r_max = 6
    else:
        radii = rng.integers(2, 4, size=(heads, nb)).astype(np.int32)
        radii[:, : nb // 3] = 1  # a cheap third: equal counts would not balance the work
        r_max = 3
    idx, cnt, maxcnt = gpu_mask(radii, shp, r_max)
    plan = torch.zeros(tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt), dtype=torch.uint8,
                       device="cuda")
    tra.tra_plan(idx, cnt, maxcnt, T, H, W, heads, 64, plan)
    torch.cuda.synchronize()
    raw = plan.cpu().numpy().view(np.int32)
    items = heads * plan_slots(T, H, W)
    cap = 2 * -(-items // 8)
    order = raw[: 8 * cap]
    lengths = raw[8 * cap: 8 * cap + 8]  # the eight range lengths follow the slots
    o_ulen = -(-(4 * (8 * cap + 8)) // 256) * 256 // 4  # then the walk lengths, 256-byte aligned
    ulen = raw[o_ulen: o_ulen + items]
    assert np.array_equal(np.sort(order[order >= 0]), np.arange(items)), "not a permutation"
    cost = np.clip(ulen, 0, min(2 * maxcnt, 8191)).astype(np.int64) + 4
    start = np.concatenate([[0], np.cumsum(cost)[:-1]])
    total = int(cost.sum())
    below = [0] + [int(np.sum(8 * start < s * total)) for s in range(1, 8)]
    lo = hi = 0
    works = []
    clamped = False
    for x in range(8):
        lo = hi
        cut = items if x == 7 else below[x + 1]
        hi = max(cut, items - cap * (7 - x))
        hi = min(max(hi, lo), min(items, lo + cap))
        clamped |= hi != cut
        col = order[x::8]
        n = hi - lo
        assert n <= cap, f"range {x} above the cap"
        assert np.array_equal(np.sort(col[:n]), np.arange(lo, hi)), f"range {x}"
        assert (col[n:] == -1).all(), f"range {x}: slots past the end"
        assert lengths[x] == n, f"range {x}: recorded length"
        # by length class (two per octave), longest class first, item order inside
        cls = np.array([order_class(v) for v in np.clip(ulen[col[:n]], 0, min(2 * maxcnt, 8191))])
        step = np.diff(cls)
        assert (step <= 0).all(), f"range {x}: not longest class first"
        assert (np.diff(col[:n])[step == 0] > 0).all(), f"range {x}: not item order in a class"
        works.append(int(cost[lo:hi].sum()))
    print(f"[order] items {items} cap {cap} range work {works} mean {total / 8:.0f} "
          f"clamped {clamped}", flush=True)
    assert hi == items
    if skewed:
        assert clamped  # the cap had to move at least one cut
    else:
        assert not clamped  # this workload fits the cap, so the cuts are the equal shares
        assert max(works) <= total / 8 + cost.max()
    # the attention along the capped order is still exact
    if skewed:
        q, k, v = ti.random_qkv(T, H, W, heads, 128, seed=23)
        out = gpu_attn(dev16(q), dev16(k), dev16(v), shp, idx, cnt, maxcnt).cpu().numpy()
        rows = item_rows(shp, 1, seed=5)
        ref = oracle.attention_rows(q, k, v, radii, rows)
        assert_close(out.reshape(-1, 128)[rows], ref, "attention along the capped order")


def plan_slots(T, H, W):
    """Item slots per head of a walk plan: vertical pairs (T ceil(nby / 2) nbx)
    or temporal pairs (ceil(T / 2) nby nbx), whichever are more."""
    nby, nbx = -(-H // 8), -(-W // 8)
    return max(T * ((nby + 1) // 2) * nbx, (T + 1) // 2 * nby * nbx)


def candidate_walk(idx_h, cnt_h, maxcnt, nb, a, b):
    """Walk length of the pair (a, b) as the union walk makes it: |A| + |B| -
    |A n B| for strictly ascending lists inside [0, nb), else |A| + |B|."""
    def lst(x):
        return [] if x < 0 else list(idx_h[x, :min(max(int(cnt_h[x]), 0), maxcnt)])

    A, B = lst(a), lst(b)

    def ascending(l):
        return all(0 <= v < nb for v in l) and all(u < v for u, v in zip(l, l[1:]))

    if B and ascending(A) and ascending(B):
        return len(A) + len(B) - len(set(A) & set(B))
    return len(A) + len(B)


def pair_table_model(idx, cnt, T, H, W):
    """The pair table the plan must hold: per head, the neighbour pairs -- the
    vertical ones (tile rows 2p, 2p + 1), or the temporal ones (one tile in
    frames 2p, 2p + 1) when their walks (candidate_walk, every fourth pair of
    either kind) take at least 5% fewer steps per list entry -- whose list lengths are within a factor of two, in raster
    order; then the other blocks sorted by length class (four per octave of
    length + 1), longest class first, raster order inside a class, paired in
    that order; then (-1, -1) up to the head's slot count.  Returns the table and
    the per-head choice (True: temporal)."""
    heads, nb = cnt.shape
    maxcnt = idx.shape[-1]
    nby, nbx = -(-H // 8), -(-W // 8)
    npy, plane = (nby + 1) // 2, nby * nbx
    slots = plan_slots(T, H, W)

    def vertical_pairs():
        for p in range(T * npy * nbx):
            t, pr, bx = p // (npy * nbx), (p // nbx) % npy, p % nbx
            qa = (t * nby + 2 * pr) * nbx + bx
            yield qa, (qa + nbx if 2 * pr + 1 < nby else -1)

    def temporal_pairs():
        for p in range((T + 1) // 2 * plane):
            tp, j = divmod(p, plane)
            qa = 2 * tp * plane + j
            yield qa, (qa + plane if 2 * tp + 1 < T else -1)

    def cls(c):
        x = max(int(c), 0) + 1
        e = x.bit_length() - 1
        f = (x >> (e - 2)) & 3 if e >= 2 else (x << (2 - e)) & 3
        return 4 * e + f

    def good(a, b):
        return 2 * min(a, b) >= max(a, b)

    table = np.full((heads, slots, 2), -1, dtype=np.int64)
    temporal = []
    for h in range(heads):
        c = np.clip(cnt[h].astype(np.int64), 0, maxcnt)
        # judged on every fourth pair of either kind: walk steps per list entry
        def steps_entries(pairs):
            u = e = 0
            for a, b in list(pairs)[::4]:
                u += candidate_walk(idx[h], cnt[h], maxcnt, nb, a, b)
                e += int(c[a]) + (int(c[b]) if b >= 0 else 0)
            return u, e

        uv, lv = steps_entries(vertical_pairs())
        ut, lt = steps_entries(temporal_pairs())
        temp = 20 * ut * lv < 19 * uv * lt
        temporal.append(temp)
        items, partner = [], {}
        for qa, qb in (temporal_pairs() if temp else vertical_pairs()):
            if qb >= 0:
                partner[qa], partner[qb] = qb, qa
            if qb < 0 or good(c[qa], c[qb]):
                items.append((qa, qb))
        orph = [b for b in range(nb) if b in partner and not good(c[b], c[partner[b]])]
        orph.sort(key=lambda b: -cls(c[b]))  # stable: raster order inside a class
        items += [(orph[i], orph[i + 1] if i + 1 < len(orph) else -1) for i in range(0, len(orph), 2)]
        table[h, :len(items)] = items
    return table, temporal


def radius_pair_table_model(radii, r_max, T, H, W):
    """The pair table of a plan built from radii (radii clamped to [0, r_max];
    radii of 127 and more rank alike).  Up to 256 tiles per frame, 1024 frames
    and 8192 blocks: vertical pairs whose radii are equal stay together; the
    other blocks are taken frame by frame, inside a frame by radius (largest
    first), tile column, tile row, and paired in that order; the items are
    listed frame by frame, each frame's kept pairs in raster order, then the
    re-paired items whose first block lies in it; then (-1, -1) up to the head's
    slot count.  Larger layers: the kept pairs in raster order, then the other
    blocks by radius (largest first) in (frame, column, row) order, paired."""
    heads, nb = radii.shape
    nby, nbx = -(-H // 8), -(-W // 8)
    plane, npy = nby * nbx, (nby + 1) // 2
    by_frame = plane <= 256 and T <= 1024 and nb <= 8192
    table = np.full((heads, plan_slots(T, H, W), 2), -1, dtype=np.int64)
    for h in range(heads):
        r = np.clip(radii[h].astype(np.int64), 0, r_max)
        kept = [[] for _ in range(T)]
        orph = []
        for f in range(T):
            for p in range(npy * nbx):
                pr, x = divmod(p, nbx)
                qa = (f * nby + 2 * pr) * nbx + x
                qb = qa + nbx if 2 * pr + 1 < nby else -1
                if qb < 0 or r[qa] == r[qb]:
                    kept[f].append((qa, qb))
            for j in range(plane):
                y, x = divmod(j, nbx)
                b = f * plane + j
                if (y ^ 1) < nby and r[b] != r[f * plane + (y ^ 1) * nbx + x]:
                    orph.append(b)
        if by_frame:
            orph.sort(key=lambda b: (b // plane, -min(r[b], 127), b % nbx, (b // nbx) % nby))
        else:
            orph.sort(key=lambda b: (-min(r[b], 127), b // plane, b % nbx, (b // nbx) % nby))
        pitems = [(orph[i], orph[i + 1] if i + 1 < len(orph) else -1) for i in range(0, len(orph), 2)]
        if by_frame:
            items, j = [], 0
            for f in range(T):
                items += kept[f]
                while j < len(pitems) and pitems[j][0] // plane == f:
                    items.append(pitems[j])
                    j += 1
        else:
            items = [it for f in range(T) for it in kept[f]] + pitems
        table[h, :len(items)] = items
    return table


def plan_pair_table(plan, T, H, W, heads, maxcnt):
    items = heads * plan_slots(T, H, W)
    rows = -(-items // 8) * 8
    cap = 2 * -(-items // 8)
    stride = -(-(2 * maxcnt) // 64) * 64
    up = lambda x: -(-x // 256) * 256
    o = up(4 * (8 * cap + 8)) + up(4 * rows) + up(4 * rows * stride)
    raw = plan.cpu().numpy()[o: o + 8 * items].view(np.int32)
    return raw.reshape(heads, -1, 2).astype(np.int64)


def temporal_lists(T, H, W, heads, seed):
    """Caller lists whose temporal neighbours (one tile in frames 2p, 2p + 1)
    nearly coincide while vertical neighbours are independent: random ascending
    lists of nb / 8 to nb / 3 blocks, the second frame of each pair keeping its
    partner's list with one block added or dropped (the last frame of an odd T
    stands alone)."""
    nby, nbx = -(-H // 8), -(-W // 8)
    plane = nby * nbx
    nb = T * plane
    rng = np.random.default_rng(seed)
    maxcnt = nb // 3 + 1
    idx = np.full((heads, nb, maxcnt), -1, dtype=np.int32)
    cnt = np.zeros((heads, nb), dtype=np.int32)
    for h in range(heads):
        for tp in range(0, T, 2):
            for j in range(plane):
                a = tp * plane + j
                la = np.sort(rng.choice(nb, size=rng.integers(nb // 8, nb // 3), replace=False))
                idx[h, a, :len(la)], cnt[h, a] = la, len(la)
                if tp + 1 < T:
                    lb = set(la.tolist())
                    x = int(rng.integers(nb))
                    lb.symmetric_difference_update({x})
                    lb = np.array(sorted(lb), dtype=np.int32)
                    idx[h, a + plane, :len(lb)], cnt[h, a + plane] = lb, len(lb)
    return idx, cnt, maxcnt


@pytest.mark.parametrize("kind", ["routing", "radii", "temporal"])
def test_pair_table(kind):
    # The plan's pair table equals the rule applied to the lists (neighbour
    # direction per head from the candidate walks, then the list lengths), every
    # query block appears in exactly one item, and attention along it is exact.
    T, H, W, heads, d = 5, 40, 56, 2, 128
    shp = (heads, T, H, W, d)
    print(f"[case] pair table {kind} {shp}", flush=True)
    nb = tra.tra_grid(T, H, W)[2]
    rng = np.random.default_rng(29)
    radii = None
    if kind == "temporal":
        li, lc, maxcnt = temporal_lists(T, H, W, heads, seed=30)
        idx, cnt = torch.from_numpy(li).cuda(), torch.from_numpy(lc).cuda()
    else:
        if kind == "routing":
            radii = np.where(rng.random((heads, nb)) < 0.2, INF, 1).astype(np.int32)
            r_max = INF
        else:
            radii = rng.integers(0, 5, size=(heads, nb)).astype(np.int32)
            r_max = 4
        idx, cnt, maxcnt = gpu_mask(radii, shp, r_max)
    plan = torch.zeros(tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt), dtype=torch.uint8,
                       device="cuda")
    tra.tra_plan(idx, cnt, maxcnt, T, H, W, heads, 64, plan)
    torch.cuda.synchronize()
    got = plan_pair_table(plan, T, H, W, heads, maxcnt)
    want, temporal = pair_table_model(idx.cpu().numpy(), cnt.cpu().numpy(), T, H, W)
    print(f"[pairs] {kind}: temporal neighbours per head {temporal}", flush=True)
    if kind == "temporal":  # lists that coincide in time take temporal neighbours
        assert all(temporal)
    assert np.array_equal(got, want), "pair table differs from the rule"
    for h in range(heads):
        blocks = got[h].ravel()
        assert np.array_equal(np.sort(blocks[blocks >= 0]), np.arange(nb)), "not a partition"
    repaired = int(np.sum(got[:, :, 1] >= 0) - 0)
    print(f"[pairs] {kind}: {repaired} two-block items of {got.shape[1] * heads} slots", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=8, family=35)
    out = torch.full(shp, float("nan"), dtype=torch.float32, device="cuda")
    tra.tra_attn_plan(dev16(q), dev16(k), dev16(v), T, H, W, heads, d, 64, plan, maxcnt, out)
    torch.cuda.synchronize()
    if radii is not None:
        ref = oracle.attention(q, k, v, radii)
    else:
        ref = oracle.attention_lists_rows(q, k, v, idx.cpu().numpy(), cnt.cpu().numpy(),
                                          np.arange(heads * T * H * W)).reshape(out.shape)
    assert_close(out.cpu().numpy(), ref, f"attention along the pair table ({kind})")


def test_binary_routing():
    # HetA-style routing: every block either local (radius 1) or dense (radius
    # infinite) from a supplied difficulty map; the mask with r_max infinite
    # gives full lists for the dense blocks (lists of 27 vs nb entries).
    T, H, W, heads, d = 6, 32, 48, 2, 128
    shp = (heads, T, H, W, d)
    print(f"[case] binary routing {shp}", flush=True)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=5, family=32)
    nb = tra.tra_grid(T, H, W)[2]
    rng = np.random.default_rng(17)
    radii = np.where(rng.random((heads, nb)) < 0.2, INF, 1).astype(np.int32)
    idx, cnt, maxcnt = gpu_mask(radii, shp, INF)
    assert maxcnt == nb
    check_lists(idx, cnt, radii, shp, maxcnt, "binary routing lists")
    c = cnt.cpu().numpy()
    assert (c[radii == INF] == nb).all()
    out = gpu_attn(dev16(q), dev16(k), dev16(v), shp, idx, cnt, maxcnt).cpu().numpy()
    rows = sample_rows(shp, 800, seed=4)
    ref = oracle.attention_rows(q, k, v, radii, rows)
    assert_close(out.reshape(-1, d)[rows], ref, "binary routing attention")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mixed", [False, True], ids=["negative", "mixed"])
def test_negative_logit_rows_on_edge_tiles(d, mixed):
    # Rows whose every logit is far below zero, on grids with ragged tiles.
    # A padded key must never stand in for such a row's max: that would push
    # every probability of the row below the fp16 range.
    for T, H, W, heads in ((3, 20, 28, 2), (2, 13, 9, 3), (2, 30, 52, 1)):
        shp = (heads, T, H, W, d)
        print(f"[case] negative logits {shp} mixed={mixed}", flush=True)
        q, k, v = ti.aligned_qkv(T, H, W, heads, d, seed=13, mixed_signs=mixed)
        qd, kd, vd = dev16(q), dev16(k), dev16(v)
        nb = tra.tra_grid(T, H, W)[2]
        radii = np.random.default_rng(4).integers(0, 3, size=(heads, nb)).astype(np.int32)
        idx, cnt, maxcnt = gpu_mask(radii, shp, 2)
        out = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
        assert_close(out, oracle.attention(q, k, v, radii), f"negative logits {shp}")
        dense = gpu_attn(qd, kd, vd, shp).cpu().numpy()
        assert_close(dense, oracle.attention(q, k, v, oracle.dense_radii(heads, nb)),
                     f"negative logits dense {shp}")


@pytest.mark.parametrize("step", [3.0, 9.0, 17.0])
def test_logits_growing_along_the_walk(step):
    # Keys whose logits grow by `step` (base 2) with every frame: along the
    # ascending walk each key tile sits above everything before it, so the
    # running reference must move when a probability would leave fp16 (17 per
    # tile: at every tile; 9: every other; 3: every sixth) and stay put in
    # between, with O and l rescaled consistently.  Dense mode and lists.
    T, H, W, heads, d = 12, 16, 16, 2, 128
    shp = (heads, T, H, W, d)
    print(f"[case] growing logits {shp} step={step}", flush=True)
    rng = np.random.default_rng(41)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    t = np.arange(T)[None, :, None, None, None]
    # q . k = a t' b with |q| = b, |k| = a t' along u: step log2 units per frame
    b = 4.0
    a = step / (np.log2(np.e) / np.sqrt(d)) / b
    q = b * u + 0.05 * rng.standard_normal((heads, T, H, W, d))
    k = (a * t) * u + 0.05 * rng.standard_normal((heads, T, H, W, d))
    v = rng.standard_normal((heads, T, H, W, d))
    q, k, v = (ti.bf16_from_f32(x.astype(np.float32)) for x in (q, k, v))
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    nb = tra.tra_grid(T, H, W)[2]
    dense = gpu_attn(qd, kd, vd, shp).cpu().numpy()
    assert_close(dense, oracle.attention(q, k, v, oracle.dense_radii(heads, nb)),
                 f"growing logits, dense, step {step}")
    radii = rng.integers(1, 6, size=(heads, nb)).astype(np.int32)
    idx, cnt, maxcnt = gpu_mask(radii, shp, 5)
    out = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
    assert_close(out, oracle.attention(q, k, v, radii), f"growing logits, lists, step {step}")


def test_mask_clamps_radius_to_r_max():
    T, H, W, heads = 6, 24, 40, 1
    shp = (heads, T, H, W, 64)
    nb = tra.tra_grid(T, H, W)[2]
    radii = np.array([[7, -2] + [1] * (nb - 2)], dtype=np.int32)
    idx, cnt, maxcnt = gpu_mask(radii, shp, 2)
    check_lists(idx, cnt, np.clip(radii, 0, 2), shp, maxcnt, "clamped radii")


def test_deterministic():
    T, H, W, heads, d = 3, 30, 52, 2, 128
    shp = (heads, T, H, W, d)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=2, family=22)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    a = gpu_attention(qd, kd, vd, shp, 1, 3).cpu().numpy()
    b = gpu_attention(qd, kd, vd, shp, 1, 3).cpu().numpy()
    assert np.array_equal(a, b)


# ------------------------------------------------- full workload shapes --

_CACHE = {}


def workload_inputs(wid):
    if wid not in _CACHE:
        _CACHE.clear()
        _CACHE[wid] = ti.make_workload_inputs(wid)
    return _CACHE[wid]


def test_wan13b_81f_every_row():
    # The headline layer in full: probe radii, lists, and every one of its
    # heads x T x H x W output rows against the oracle on the GPU's radii.
    c = ti.WORKLOADS[ti.WAN13B_81F]
    shp = (c.heads, c.T, c.H, c.W, c.d)
    print(f"[case] {c.slug} every row {shp} r=[{c.r_min},{c.r_max}]", flush=True)
    q, k, v = workload_inputs(ti.WAN13B_81F)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    hn_g, r_g = gpu_probe(qd, kd, shp, c.r_min, c.r_max)
    hn_o, r_o = oracle.probe(q, k, c.r_min, c.r_max)
    check_radii(hn_g, r_g, hn_o, r_o, c.r_min, c.r_max, f"{c.slug} probe")
    idx, cnt, maxcnt = gpu_mask(r_g, shp, c.r_max)
    check_lists(idx, cnt, r_g, shp, maxcnt, f"{c.slug} mask")
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    print(f"[parity] {c.slug}: block density {cnt.sum().item() / (c.heads * nb * nb):.4f}",
          flush=True)
    staged = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
    del idx, cnt
    got = gpu_attention(qd, kd, vd, shp, c.r_min, c.r_max).cpu().numpy()
    # the fused call builds its walks from the radii without the lists: the
    # same walks, so the same bits as the staged calls
    assert np.array_equal(got, staged), f"{c.slug}: fused call differs from the staged calls"
    del staged
    ref = oracle.attention(q, k, v, r_g)
    assert_close(got, ref, f"{c.slug} attention (all {c.heads * c.N} rows)")


def test_wan13b_81f_dense_mode():
    c = ti.WORKLOADS[ti.WAN13B_81F]
    shp = (c.heads, c.T, c.H, c.W, c.d)
    print(f"[case] {c.slug} dense {shp}", flush=True)
    q, k, v = workload_inputs(ti.WAN13B_81F)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    out = gpu_attention(qd, kd, vd, shp, INF, INF)
    # two rows of every query block (one per wave where the block has more
    # than 32 real queries): every work item of the dense launch
    rows = np.union1d(item_rows(shp, 2, seed=11), sample_rows(shp, 0, seed=11))
    got = out.view(-1, c.d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    ref = oracle.attention_rows(q, k, v, oracle.dense_radii(c.heads, nb), rows)
    assert_close(got, ref, f"{c.slug} dense ({rows.size} rows, every query block)")


@pytest.mark.parametrize("wid", [ti.WAN13B_241F, ti.WAN14B_81F, ti.HUNYUAN_129F],
                         ids=lambda w: ti.WORKLOADS[w].slug)
def test_full_workload(wid):
    # The larger layers: probe, lists in full; outputs on one random row of
    # every query block (so every work item and walk of the launch is
    # compared) plus edge-tile rows.
    c = ti.WORKLOADS[wid]
    shp = (c.heads, c.T, c.H, c.W, c.d)
    print(f"[case] {c.slug} {shp} r=[{c.r_min},{c.r_max}]", flush=True)
    q, k, v = workload_inputs(wid)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    hn_g, r_g = gpu_probe(qd, kd, shp, c.r_min, c.r_max)
    hn_o, r_o = oracle.probe(q, k, c.r_min, c.r_max)
    check_radii(hn_g, r_g, hn_o, r_o, c.r_min, c.r_max, f"{c.slug} probe")
    idx, cnt, maxcnt = gpu_mask(r_g, shp, c.r_max)
    check_lists(idx, cnt, r_g, shp, maxcnt, f"{c.slug} mask")
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    density = cnt.sum().item() / (c.heads * nb * nb)
    print(f"[parity] {c.slug}: block density {density:.4f}", flush=True)
    staged = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt)
    del idx, cnt
    out = gpu_attention(qd, kd, vd, shp, c.r_min, c.r_max)
    assert torch.equal(out, staged), f"{c.slug}: fused call differs from the staged calls"
    del staged
    rows = np.union1d(item_rows(shp, 1, seed=wid), sample_rows(shp, 0, seed=wid))
    got = out.view(-1, c.d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    del out
    ref = oracle.attention_rows(q, k, v, r_g, rows)
    assert_close(got, ref, f"{c.slug} attention ({rows.size} rows, every query block)")


# ------------------------------------------------------- the range of V --

@pytest.mark.parametrize("d", [64, 128])
def test_v_of_any_finite_magnitude(d):
    # V enters the fp16 P.V product scaled by a power of two per head: heads
    # whose values reach 1e5 (beyond fp16's 65504) or stay near 1e-6 (below
    # fp16's normal range), and one head mixing both extremes, must all match
    # the oracle within the usual bars (dense mode and lists).
    T, H, W, heads = 3, 20, 28, 4
    shp = (heads, T, H, W, d)
    print(f"[case] V magnitudes {shp}", flush=True)
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=31)
    vf = ti.bf16_to_f32(v).astype(np.float64)
    scale = np.array([1e5 / 4.5, 1e-6, 1.0, 1.0])[:, None, None, None, None]
    vf = vf * scale
    # head 3: a few values at 1e5 among N(0, 1) values and values near 1e-6
    rng = np.random.default_rng(2)
    flat = vf[3].reshape(-1)
    pick = rng.choice(flat.size, size=64, replace=False)
    flat[pick[:8]] = 1e5 * np.sign(rng.standard_normal(8))
    flat[pick[8:]] = 1e-6 * rng.standard_normal(56)
    v2 = ti.bf16_from_f32(vf.astype(np.float32))
    vmax = np.abs(ti.bf16_to_f32(v2)).reshape(heads, -1).max(axis=1)
    print(f"[case] per-head max|v| {vmax}", flush=True)
    assert vmax[0] > 65504 and vmax[1] < 6.1e-5
    qd, kd, vd = dev16(q), dev16(k), dev16(v2)
    nb = tra.tra_grid(T, H, W)[2]
    dense = gpu_attn(qd, kd, vd, shp).cpu().numpy()
    ref = oracle.attention(q, k, v2, oracle.dense_radii(heads, nb))
    assert_close(dense[2], ref[2], "dense, head 2 (N(0, 1) values)")
    # Every head against the L1-relative bar, and the max-abs bar in units of
    # the head's value scale: max|v| / 4 (about 1 for N(0, 1) values, whose
    # largest |v| over a head is 4 to 5).  fp16 probabilities carry a relative
    # rounding of 2^-12 whatever V is, so an output row that averages values
    # of 1e5 has an absolute error of order 1e5 2^-12 and only such a bar is
    # scale-free.
    bar = MAX_ABS * vmax / 4.0
    for h in range(heads):
        err = np.abs(dense[h].astype(np.float64) - ref[h])
        print(f"[parity] V magnitudes dense head {h}: max_abs={err.max():.3e} (bar {bar[h]:.3e}) "
              f"l1_rel={err.sum() / np.abs(ref[h]).sum():.3e}", flush=True)
        assert np.isfinite(dense[h]).all()
        assert err.sum() / np.abs(ref[h]).sum() <= L1_REL
        assert err.max() <= bar[h]
    radii = np.random.default_rng(3).integers(0, 3, size=(heads, nb)).astype(np.int32)
    idx, cnt, maxcnt = gpu_mask(radii, shp, 2)
    sparse = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt).cpu().numpy()
    ref = oracle.attention(q, k, v2, radii)
    for h in range(heads):
        err = np.abs(sparse[h].astype(np.float64) - ref[h])
        assert np.isfinite(sparse[h]).all()
        assert err.sum() / np.abs(ref[h]).sum() <= L1_REL, f"lists, head {h}"
        assert err.max() <= bar[h], f"lists, head {h}"
    # the fused layer (probe radii) over the same values
    out = gpu_attention(qd, kd, vd, shp, 0, 2).cpu().numpy()
    hn_g, r_g = gpu_probe(qd, kd, shp, 0, 2)
    ref = oracle.attention(q, k, v2, r_g)
    for h in range(heads):
        err = np.abs(out[h].astype(np.float64) - ref[h])
        assert np.isfinite(out[h]).all()
        assert err.sum() / np.abs(ref[h]).sum() <= L1_REL, f"layer, head {h}"
        assert err.max() <= bar[h], f"layer, head {h}"


# ------------------------------------------------- workspace and timing --

def test_probe_with_caller_workspace():
    # tra_probe with a caller-owned workspace of tra_workspace_bytes bytes gives
    # the same bits as with library scratch, and writes nothing past it.
    T, H, W, heads, d = 3, 20, 28, 2, 128
    shp = (heads, T, H, W, d)
    q, k, _ = ti.make_inputs(T, H, W, heads, d, seed=4, family=33)
    qd, kd = dev16(q), dev16(k)
    nb = tra.tra_grid(T, H, W)[2]
    nbytes = tra.tra_workspace_bytes(T, H, W, heads, d, 64, 3)
    guard = 4096
    ws = torch.full((nbytes + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    r1 = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    h1 = torch.empty(heads, nb, dtype=torch.float32, device="cuda")
    tra.tra_probe(qd, kd, T, H, W, heads, d, 64, 0, 3, r1, h1, ws=ws)
    hn_g, r_g = gpu_probe(qd, kd, shp, 0, 3)
    torch.cuda.synchronize()
    assert np.array_equal(r1.cpu().numpy(), r_g)
    assert np.array_equal(h1.cpu().numpy(), hn_g)
    assert (ws[nbytes:].cpu().numpy() == 0x5A).all(), "wrote past the workspace"


def test_timed_attention_matches_attention():
    # The benchmark helper runs the same kernel: its output equals tra_attn's,
    # for lists and for the dense mode.
    T, H, W, heads, d = 4, 24, 40, 2, 128
    shp = (heads, T, H, W, d)
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=6, family=34)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    nb = tra.tra_grid(T, H, W)[2]
    radii = np.random.default_rng(8).integers(0, 3, size=(heads, nb)).astype(np.int32)
    idx, cnt, maxcnt = gpu_mask(radii, shp, 2)
    for lists in (True, False):
        out = torch.full(shp, float("nan"), dtype=torch.float32, device="cuda")
        ms = tra.tra_time_attn(qd, kd, vd, T, H, W, heads, d, 64, idx if lists else None,
                               cnt if lists else None, None, maxcnt if lists else 0, 3, out)
        ref = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt) if lists else gpu_attn(qd, kd, vd, shp)
        assert ms > 0.0
        assert torch.equal(out, ref)
    # along a stored plan (from the radii) and in dense mode without a plan
    plan = torch.empty(tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt), dtype=torch.uint8,
                       device="cuda")
    tra.tra_plan_radius(torch.from_numpy(radii).cuda(), T, H, W, heads, 64, 2, plan)
    for planned in (True, False):
        out = torch.full(shp, float("nan"), dtype=torch.float32, device="cuda")
        ms = tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan if planned else None,
                                    maxcnt if planned else 0, 3, out)
        ref = gpu_attn(qd, kd, vd, shp, idx, cnt, maxcnt) if planned else gpu_attn(qd, kd, vd, shp)
        assert ms > 0.0
        assert torch.equal(out, ref)
