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
    print(f"[parity] {what}: h_norm max|d|={np.abs(hn_gpu - hn_ref).max():.2e}, "
          f"boundary blocks={int(band.sum())}, radius mismatches={int(diff.sum())}", flush=True)
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
    # Each attention work item walks the union of a vertically adjacent pair
    # of query blocks' lists: ascending lists merge (overlaps computed once,
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


def test_work_order_ranges():
    # The work order deals the walk items to eight XCD ranges: contiguous raster
    # ranges cut at equal shares of the total work (walk length + 4 per item),
    # each of at most cap = 2 ceil(items / 8) items, taken longest first into
    # grid slots 8 k + x, -1 past a range's end.  Every item appears once.
    T, H, W, heads = 6, 30, 52, 3
    shp = (heads, T, H, W, 128)
    print(f"[case] work order {shp}", flush=True)
    nb = tra.tra_grid(T, H, W)[2]
    rng = np.random.default_rng(17)
    radii = rng.integers(2, 4, size=(heads, nb)).astype(np.int32)
    radii[:, : nb // 3] = 1  # a cheap third: equal counts would not balance the work
    idx, cnt, maxcnt = gpu_mask(radii, shp, 3)
    plan = torch.zeros(tra.tra_plan_bytes(T, H, W, heads, 64, maxcnt), dtype=torch.uint8,
                       device="cuda")
    tra.tra_plan(idx, cnt, maxcnt, T, H, W, heads, 64, plan)
    torch.cuda.synchronize()
    raw = plan.cpu().numpy().view(np.int32)
    nby, nbx = -(-H // 8), -(-W // 8)
    items = heads * T * ((nby + 1) // 2) * nbx
    cap = 2 * -(-items // 8)
    order = raw[: 8 * cap]
    o_ulen = -(-(4 * 8 * cap) // 256) * 256 // 4  # the walk lengths follow, 256-byte aligned
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
        assert np.array_equal(np.sort(col[:n]), np.arange(lo, hi)), f"range {x}"
        assert (col[n:] == -1).all(), f"range {x}: slots past the end"
        assert (np.diff(ulen[col[:n]]) <= 0).all(), f"range {x}: not longest first"
        works.append(int(cost[lo:hi].sum()))
    print(f"[order] items {items} cap {cap} range work {works} mean {total / 8:.0f} "
          f"clamped {clamped}", flush=True)
    assert not clamped  # this workload fits the cap, so the cuts are the equal shares
    assert max(works) <= total / 8 + cost.max()


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


@pytest.mark.parametrize("wid", [ti.WAN13B_81F, ti.WAN13B_241F, ti.WAN14B_81F, ti.HUNYUAN_129F],
                         ids=lambda w: ti.WORKLOADS[w].slug)
def test_full_workload(wid):
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
    del idx, cnt
    out = gpu_attention(qd, kd, vd, shp, c.r_min, c.r_max)
    rows = sample_rows(shp, 96, seed=wid)
    got = out.view(-1, c.d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    del out
    ref = oracle.attention_rows(q, k, v, r_g, rows)
    assert_close(got, ref, f"{c.slug} attention (sampled rows)")


def test_wan13b_81f_dense_mode():
    c = ti.WORKLOADS[ti.WAN13B_81F]
    shp = (c.heads, c.T, c.H, c.W, c.d)
    print(f"[case] {c.slug} dense {shp}", flush=True)
    q, k, v = workload_inputs(ti.WAN13B_81F)
    qd, kd, vd = dev16(q), dev16(k), dev16(v)
    out = gpu_attention(qd, kd, vd, shp, INF, INF)
    rows = sample_rows(shp, 48, seed=11)
    got = out.view(-1, c.d)[torch.from_numpy(rows).cuda()].cpu().numpy()
    nb = tra.tra_grid(c.T, c.H, c.W)[2]
    ref = oracle.attention_rows(q, k, v, oracle.dense_radii(c.heads, nb), rows)
    assert_close(got, ref, f"{c.slug} dense (sampled rows)")
