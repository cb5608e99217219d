"""Pins of the fp64 CPU oracle against things other than itself.

The pages print no worked example, so each oracle function is pinned by
brute force on tiny grids, closed forms, invariants, or library routines
(torch's scaled-dot-product attention in fp64, scipy's softmax and entropy).
Block membership in these tests is built by slicing tiles out of the grid,
not by the oracle's coordinate arithmetic.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch
import torch.nn.functional as F

import oracle
import tra_inputs as ti

INF = oracle.RADIUS_INF


# ---------------------------------------------------------------- helpers --

def tile_membership(T, H, W, s=8):
    """Block id per token (raster order) and block coordinates, built by slicing."""
    nby, nbx = -(-H // s), -(-W // s)
    ids = np.full((T, H, W), -1, dtype=np.int64)
    coords = []
    b = 0
    for t in range(T):
        for by in range(nby):
            for bx in range(nbx):
                ids[t, by * s:(by + 1) * s, bx * s:(bx + 1) * s] = b
                coords.append((t, by, bx))
                b += 1
    assert (ids >= 0).all()
    return ids.ravel(), np.array(coords, dtype=np.int64)


def token_mask(T, H, W, radii_of_blocks, s=8):
    """Explicit N x N token mask from tile membership: brute force."""
    ids, coords = tile_membership(T, H, W, s)
    bc = coords[ids]  # (N, 3) block coordinates of each token
    dist = np.abs(bc[:, None, :] - bc[None, :, :]).max(axis=2)
    r = np.asarray(radii_of_blocks, dtype=np.int64)[ids]
    return dist <= r[:, None]


def f64(x):
    return ti.bf16_to_f32(x).astype(np.float64)


def sdpa(q, k, v, mask=None):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m).numpy()


# ------------------------------------------------------------------- pool --

def test_pool_matches_tile_slices():
    q, _, _ = ti.random_qkv(3, 13, 19, 2, 16, seed=3)
    got = oracle.pool(q)
    x = f64(q)
    nby, nbx = 2, 3
    b = 0
    for t in range(3):
        for by in range(nby):
            for bx in range(nbx):
                ref = x[:, t, 8 * by:8 * by + 8, 8 * bx:8 * bx + 8, :].mean(axis=(1, 2))
                np.testing.assert_allclose(got[:, b], ref, rtol=0, atol=1e-12)
                b += 1


def test_pool_ragged_tiles_ignore_pad_cells():
    # a constant value per block: the mean over real tokens is that constant,
    # whatever the number of real tokens in the tile (10x11 grid -> 2x2 ragged tiles)
    T, H, W, d = 2, 10, 11, 4
    ids, _ = tile_membership(T, H, W)
    vals = (np.arange(ids.max() + 1, dtype=np.float32) + 1.0)[ids]
    x = np.repeat(vals[:, None], d, axis=1).reshape(1, T, H, W, d)
    got = oracle.pool(ti.bf16_from_f32(x))
    np.testing.assert_array_equal(got[0, :, 0], np.arange(ids.max() + 1) + 1.0)


# ------------------------------------------------------------------ probe --

def test_radius_quantiser_closed_form():
    # R = r_max - r_min + 1 = 8; boundaries at k/8 (exact binary fractions)
    assert oracle.radius(0.0, 1, 8) == 1
    for kk in range(8):
        assert oracle.radius(kk / 8, 1, 8) == 1 + kk
        assert oracle.radius(kk / 8 + 1e-5, 1, 8) == 1 + kk
        if kk:
            assert oracle.radius(kk / 8 - 1e-5, 1, 8) == kk
    assert oracle.radius(1.0, 1, 8) == 8          # clamp at H_norm = 1
    assert oracle.radius(0.5, 3, 3) == 3          # r_min = r_max: constant radius
    assert oracle.radius(0.999999, 0, 16) == 16
    assert oracle.radius(0.3, INF, INF) == INF    # dense


def test_probe_entropy_matches_scipy():
    T, H, W, heads, d = 4, 12, 20, 2, 32
    q, k, _ = ti.make_inputs(T, H, W, heads, d, seed=0, family=11)
    hn, r = oracle.probe(q, k, 1, 8)
    ids, coords = tile_membership(T, H, W)
    nb = len(coords)
    for h in range(heads):
        xq = f64(q[h]).reshape(-1, d)
        xk = f64(k[h]).reshape(-1, d)
        qb = np.stack([xq[ids == b].mean(axis=0) for b in range(nb)])
        kb = np.stack([xk[ids == b].mean(axis=0) for b in range(nb)])
        logits = qb @ kb.T / math.sqrt(d)
        p = scipy.special.softmax(logits, axis=1)
        Hs = scipy.stats.entropy(p, axis=1)
        np.testing.assert_allclose(hn[h], Hs / math.log(nb), rtol=0, atol=1e-12)
        # radii follow the quantiser of the same entropies
        assert all(r[h, b] == oracle.radius(hn[h, b], 1, 8) for b in range(nb))


def test_probe_zero_queries_give_uniform_entropy_and_r_max():
    q, k, _ = ti.random_qkv(3, 16, 16, 2, 16, seed=5)
    q[:] = 0
    hn, r = oracle.probe(q, k, 2, 6)
    np.testing.assert_allclose(hn, 1.0, atol=1e-12)
    assert (r == 6).all()


def _two_level_inputs(a_vals, T=6, H=8, W=16, d=64):
    """Block c of k = e_c (one-hot); block b of q = a_b * sqrt(d) * e_b.

    Then the pooled logits are s_bc = a_b * [b == c]: one logit a_b, the rest 0.
    """
    ids, coords = tile_membership(T, H, W)
    nb = len(coords)
    assert nb <= d and len(a_vals) == nb
    kx = np.zeros((T * H * W, d), dtype=np.float32)
    qx = np.zeros_like(kx)
    kx[np.arange(T * H * W), ids] = 1.0
    qx[np.arange(T * H * W), ids] = np.asarray(a_vals, dtype=np.float32)[ids] * math.sqrt(d)
    q = ti.bf16_from_f32(qx.reshape(1, T, H, W, d))
    k = ti.bf16_from_f32(kx.reshape(1, T, H, W, d))
    a_exact = ti.bf16_to_f32(ti.bf16_from_f32(np.asarray(a_vals, np.float32) * math.sqrt(d))) / math.sqrt(d)
    return q, k, nb, a_exact.astype(np.float64)


def test_probe_two_level_logits_closed_form():
    nb = 12
    a_vals = np.linspace(-3.0, 9.0, nb)
    q, k, nb, a = _two_level_inputs(a_vals)
    hn, r = oracle.probe(q, k, 0, 5)
    Z = np.exp(a) + nb - 1
    Hc = np.log(Z) - a * np.exp(a) / Z
    np.testing.assert_allclose(hn[0], Hc / math.log(nb), rtol=0, atol=1e-13)
    R = 6
    for b in range(nb):
        x = Hc[b] / math.log(nb) * R
        if abs(x - round(x)) > 1e-9:
            assert r[0, b] == min(int(math.floor(x)), 5)


def test_probe_huge_self_logit_gives_r_min():
    q, k, nb, a = _two_level_inputs(np.full(12, 60.0))
    hn, r = oracle.probe(q, k, 2, 9)
    assert (hn < 1e-20).all()
    assert (r == 2).all()


def test_probe_single_block_grid():
    q, k, _ = ti.random_qkv(1, 5, 7, 2, 8, seed=1)
    hn, r = oracle.probe(q, k, 1, 4)
    assert hn.shape == (2, 1) and (hn == 0).all() and (r == 1).all()


def test_probe_dense_and_errors():
    q, k, _ = ti.random_qkv(2, 8, 8, 1, 8, seed=1)
    hn, r = oracle.probe(q, k, INF, INF)
    assert (r == INF).all()
    with pytest.raises(ValueError):
        oracle.probe(q, k, 3, 2)
    with pytest.raises(ValueError):
        oracle.probe(q, k, -1, 2)


# ------------------------------------------------------------ block lists --

@pytest.mark.parametrize("seed", range(6))
def test_block_lists_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, H, W = (int(x) for x in rng.integers(1, 13, size=3) * np.array([1, 2, 2]))
    ids, coords = tile_membership(T, H, W)
    nb = len(coords)
    heads = 2
    radii = rng.integers(0, 4, size=(heads, nb)).astype(np.int32)
    idx, cnt = oracle.block_lists(radii, T, H, W)
    for h in range(heads):
        M = token_mask(T, H, W, radii[h])
        # kb in L(qb) iff some token pair (i in qb, j in kb) is kept
        blk_any = np.zeros((nb, nb), dtype=bool)
        for b in range(nb):
            rows = M[ids == b]
            kept_tokens = rows.any(axis=0)
            blk_any[b, np.unique(ids[kept_tokens])] = True
        for b in range(nb):
            ref = np.flatnonzero(blk_any[b])
            assert cnt[h, b] == ref.size
            np.testing.assert_array_equal(idx[h, b, :cnt[h, b]], ref)


def test_block_lists_closed_form_counts_and_invariants():
    T, H, W = 9, 30, 52
    nby, nbx, nb = oracle.grid_blocks(T, H, W)
    for r0 in [0, 1, 2, 5, INF]:
        radii = np.full((1, nb), r0, dtype=np.int32)
        idx, cnt = oracle.block_lists(radii, T, H, W)
        rr = min(r0, 10 ** 6)
        for b in range(nb):
            t, by, bx = b // (nby * nbx), (b // nbx) % nby, b % nbx
            closed = 1
            for c, n in ((t, T), (by, nby), (bx, nbx)):
                closed *= min(c + rr, n - 1) - max(c - rr, 0) + 1
            assert cnt[0, b] == closed
            row = idx[0, b, :cnt[0, b]]
            assert b in row                       # own block always kept
            assert (np.diff(row) > 0).all()      # strictly ascending
        # symmetric when all radii are equal
        A = np.zeros((nb, nb), dtype=bool)
        for b in range(nb):
            A[b, idx[0, b, :cnt[0, b]]] = True
        assert (A == A.T).all()


def test_block_lists_overflow_is_an_error():
    radii = np.full((1, 8), 3, dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.block_lists(radii, 8, 8, 8, maxcnt=4)


# -------------------------------------------------------------- attention --

def test_attention_dense_equals_textbook_attention():
    T, H, W, heads, d = 3, 10, 13, 2, 32
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=2)
    nb = oracle.grid_blocks(T, H, W)[2]
    got = oracle.attention(q, k, v, oracle.dense_radii(heads, nb))
    ref = sdpa(f64(q).reshape(heads, -1, d), f64(k).reshape(heads, -1, d), f64(v).reshape(heads, -1, d))
    np.testing.assert_allclose(got.reshape(heads, -1, d), ref, rtol=0, atol=1e-12)
    # a finite radius covering the whole grid is the same thing
    got2 = oracle.attention(q, k, v, np.full((heads, nb), 3, dtype=np.int32))
    np.testing.assert_allclose(got2, got, rtol=0, atol=1e-13)


def test_attention_radius0_is_per_tile_attention():
    T, H, W, heads, d = 2, 11, 17, 2, 16
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=4)
    nb = oracle.grid_blocks(T, H, W)[2]
    got = oracle.attention(q, k, v, np.zeros((heads, nb), dtype=np.int32))
    xq, xk, xv = f64(q), f64(k), f64(v)
    for t in range(T):
        for by in range(2):
            for bx in range(3):
                sl = (slice(None), t, slice(8 * by, 8 * by + 8), slice(8 * bx, 8 * bx + 8))
                tq, tk, tv = (a[sl].reshape(heads, -1, d) for a in (xq, xk, xv))
                ref = sdpa(tq, tk, tv)
                np.testing.assert_allclose(got[sl].reshape(heads, -1, d), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_attention_random_radii_vs_masked_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    T, H, W, heads, d = 5, 14, 18, 2, 16
    q, k, v = ti.make_inputs(T, H, W, heads, d, seed=seed, family=12)
    nb = oracle.grid_blocks(T, H, W)[2]
    radii = rng.integers(0, 3, size=(heads, nb)).astype(np.int32)
    got = oracle.attention(q, k, v, radii)
    for h in range(heads):
        M = token_mask(T, H, W, radii[h])
        ref = sdpa(f64(q[h]).reshape(1, -1, d), f64(k[h]).reshape(1, -1, d), f64(v[h]).reshape(1, -1, d),
                   mask=M[None])
        np.testing.assert_allclose(got[h].reshape(-1, d), ref[0], rtol=0, atol=1e-12)


def test_attention_weights_sum_to_one():
    # v constant across tokens: every output row equals that constant
    T, H, W, heads, d = 3, 12, 9, 2, 8
    q, k, _ = ti.random_qkv(T, H, W, heads, d, seed=6, scale=3.0)
    c = ti.bf16_from_f32(np.linspace(-2, 2, d).astype(np.float32))
    v = np.broadcast_to(c, q.shape).copy()
    nb = oracle.grid_blocks(T, H, W)[2]
    radii = np.random.default_rng(0).integers(0, 2, size=(heads, nb)).astype(np.int32)
    got = oracle.attention(q, k, v, radii)
    np.testing.assert_allclose(got, np.broadcast_to(f64(c), got.shape), rtol=0, atol=1e-13)


def test_attention_rows_agree_with_full():
    T, H, W, heads, d = 3, 9, 10, 2, 16
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=8)
    nb = oracle.grid_blocks(T, H, W)[2]
    radii = np.random.default_rng(1).integers(0, 2, size=(heads, nb)).astype(np.int32)
    full = oracle.attention(q, k, v, radii).reshape(heads * T * H * W, d)
    rows = np.array([0, 5, 77, 269, 270, 539])
    np.testing.assert_array_equal(oracle.attention_rows(q, k, v, radii, rows), full[rows])


# ------------------------------------------------ token-level radius policy --

def test_token_entropy_matches_scipy():
    T, H, W, heads, d = 2, 8, 12, 2, 16
    q, k, _ = ti.random_qkv(T, H, W, heads, d, seed=21, scale=2.0)
    got = oracle.token_entropy(q, k).reshape(heads, -1)
    qf, kf = f64(q).reshape(heads, -1, d), f64(k).reshape(heads, -1, d)
    for h in range(heads):
        p = scipy.special.softmax(qf[h] @ kf[h].T / math.sqrt(d), axis=1)
        np.testing.assert_allclose(got[h], scipy.stats.entropy(p, axis=1), rtol=1e-12, atol=1e-12)


def test_token_entropy_closed_forms():
    T, H, W, heads, d = 2, 5, 7, 1, 16
    N = T * H * W
    q, _, _ = ti.random_qkv(T, H, W, heads, d, seed=22)
    k0 = np.zeros_like(q)  # every logit 0: uniform rows
    np.testing.assert_allclose(oracle.token_entropy(q, k0), math.log(N), rtol=1e-13)
    # one dominant key: a logit of 100 * 100 / 4 against zeros -> a one-hot row
    big = int(ti.bf16_from_f32(np.array([100.0], dtype=np.float32))[0])
    qb = np.zeros_like(q)
    qb[..., 0] = big
    kb = np.zeros_like(q)
    kb[0, 1, 2, 3, 0] = big
    assert np.abs(oracle.token_entropy(qb, kb)).max() < 1e-12


def test_token_radius_closed_forms():
    rng = np.random.default_rng(3)
    T, H, W, heads = 5, 4, 6, 2
    N = T * H * W
    ent = rng.uniform(0.0, math.log(N), size=(heads, T, H, W))
    tau = 0.7
    b = np.clip(tau * np.exp(ent), 1.0, N)
    # no temporal decay: the disk has the same area in all T frames
    np.testing.assert_allclose(oracle.token_radius(ent, tau, 0.0), np.sqrt(b / (math.pi * T)),
                               rtol=1e-14)
    # with decay, the disks' areas over the frames add up to the budget
    gamma = 0.35
    r0 = oracle.token_radius(ent, tau, gamma)
    t = np.arange(T)
    for ti_ in range(T):
        area = (math.pi * (r0[:, ti_][..., None] * np.exp(-gamma * np.abs(t - ti_))) ** 2).sum(-1)
        np.testing.assert_allclose(area, b[:, ti_], rtol=1e-12)
    # budget clamps: at least one key, at most all N
    one = oracle.token_radius(np.zeros((1, 1, 3, 3)), 1e-9, 0.0)
    np.testing.assert_allclose(one, math.sqrt(1.0 / math.pi), rtol=1e-14)
    alln = oracle.token_radius(np.full((1, 1, 3, 3), 50.0), 1.0, 0.0)
    np.testing.assert_allclose(alln, math.sqrt(9.0 / math.pi), rtol=1e-14)


def lists_of(idx, cnt):
    return [idx[n, :cnt[n]].tolist() for n in range(len(cnt))]


def test_token_lists_geometry_by_hand():
    # two tiles side by side (x 0..7 | 8..15): the closest tokens are 1 apart
    r = np.full((1, 1, 8, 16), 1.0)
    assert lists_of(*oracle.token_lists(r, 0.0)) == [[0, 1], [0, 1]]
    assert lists_of(*oracle.token_lists(r * 0.99, 0.0)) == [[0], [1]]
    # one token of the left tile reaches across: one vote
    r = np.full((1, 1, 8, 16), 0.1)
    r[0, 0, 3, 7] = 1.0
    assert lists_of(*oracle.token_lists(r, 0.0, min_votes=1)) == [[0, 1], [1]]
    assert lists_of(*oracle.token_lists(r, 0.0, min_votes=2)) == [[0], [1]]
    # 2 x 2 tiles: the diagonal tile is sqrt(2) away (Euclidean, not Chebyshev)
    r = np.full((1, 1, 16, 16), 1.0)
    assert lists_of(*oracle.token_lists(r, 0.0))[0] == [0, 1, 2]
    assert lists_of(*oracle.token_lists(r * 1.42, 0.0))[0] == [0, 1, 2, 3]
    assert lists_of(*oracle.token_lists(r * 1.41, 0.0))[0] == [0, 1, 2]


def test_token_lists_decay_and_query_frame_radius():
    # two tiles side by side per frame, 3 frames: radius 1 reaches the
    # neighbouring tile in its own frame; decayed to exp(-0.1) < 1 it does not
    # in the next frames (the co-located tiles stay)
    r = np.full((1, 3, 8, 16), 1.0)
    lists = lists_of(*oracle.token_lists(r, 0.1))
    assert lists[2] == [0, 2, 3, 4]
    assert lists[0] == [0, 1, 2, 4]
    assert lists_of(*oracle.token_lists(r, 0.0))[2] == [0, 1, 2, 3, 4, 5]
    # the radius is the query token's, whatever frame the key lies in
    r = np.full((1, 2, 8, 16), 0.1)
    r[0, 0] = 1.0
    lists = lists_of(*oracle.token_lists(r, 0.0))
    assert lists[0] == [0, 1, 2, 3]
    assert lists[2] == [0, 2]


def test_token_lists_temporal_reach_and_extremes():
    # one tile per frame: a shrinking disk still holds the co-located token, so
    # every frame's tile is kept however small the radius or fast the decay
    r = np.full((1, 3, 8, 8), 0.01)
    for gamma in (0.0, 5.0):
        assert lists_of(*oracle.token_lists(r, gamma)) == [[0, 1, 2]] * 3
    # tiny radii on a larger grid: exactly the co-located tile of each frame
    T, H, W = 3, 16, 24
    idx, cnt = oracle.token_lists(np.full((1, T, H, W), 0.3), 1.0)
    nb = oracle.grid_blocks(T, H, W)[2]
    per = nb // T
    assert (cnt == T).all()
    assert lists_of(idx, cnt)[4] == [4 % per + per * t for t in range(T)]
    # huge radii without decay: everything
    idx, cnt = oracle.token_lists(np.full((1, T, H, W), 100.0), 0.0)
    assert (cnt == nb).all()
    # votes needed beyond the real tokens of a partial tile: nothing kept
    idx, cnt = oracle.token_lists(np.full((1, 1, 5, 8), 100.0), 0.0, min_votes=41)
    assert (cnt == 0).all()
    idx, cnt = oracle.token_lists(np.full((1, 1, 5, 8), 100.0), 0.0, min_votes=40)
    assert (cnt == 1).all()


def test_token_lists_symmetric_and_monotone():
    rng = np.random.default_rng(8)
    T, H, W = 3, 16, 16
    nb = oracle.grid_blocks(T, H, W)[2]
    r = np.full((1, T, H, W), 6.5)
    idx, cnt = oracle.token_lists(r, 0.4)
    keep = np.zeros((nb, nb), dtype=bool)
    for q_, l in enumerate(lists_of(idx, cnt)):
        keep[q_, l] = True
    assert (keep == keep.T).all() and keep.diagonal().all()
    r = rng.uniform(0.5, 9.0, size=(2, T, H, W))
    small = lists_of(*oracle.token_lists(r, 0.3, r2_scale=0.9))
    big = lists_of(*oracle.token_lists(r, 0.3, r2_scale=1.1))
    assert all(set(a) <= set(b) for a, b in zip(small, big))


def block_key_mask(T, H, W, lists):
    """N x N mask: key j kept for query i iff block(j) is in block(i)'s list."""
    ids, _ = tile_membership(T, H, W)
    nb = ids.max() + 1
    keep = np.zeros((nb, nb), dtype=bool)
    for b, l in enumerate(lists):
        keep[b, l] = True
    return keep[ids][:, ids]


def test_attention_lists_vs_masked_sdpa():
    T, H, W, heads, d = 2, 12, 16, 1, 8
    q, k, v = ti.random_qkv(T, H, W, heads, d, seed=24)
    nb = oracle.grid_blocks(T, H, W)[2]
    rng = np.random.default_rng(5)
    lists = [sorted(set([b] + rng.choice(nb, size=rng.integers(0, nb), replace=False).tolist()))
             for b in range(nb)]
    maxcnt = nb
    idx = np.full((1, nb, maxcnt), -1, dtype=np.int32)
    cnt = np.zeros((1, nb), dtype=np.int32)
    for b, l in enumerate(lists):
        idx[0, b, :len(l)] = l
        cnt[0, b] = len(l)
    rows = np.arange(T * H * W)
    got = oracle.attention_lists_rows(q, k, v, idx, cnt, rows)
    mask = block_key_mask(T, H, W, lists)
    ref = sdpa(f64(q).reshape(1, -1, d), f64(k).reshape(1, -1, d), f64(v).reshape(1, -1, d), mask)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # every entry twice: uniform doubling of the weights leaves the softmax unchanged
    idx2 = np.full((1, nb, 2 * maxcnt), -1, dtype=np.int32)
    for b, l in enumerate(lists):
        idx2[0, b, :2 * len(l)] = l + l
    got2 = oracle.attention_lists_rows(q, k, v, idx2, 2 * cnt, rows)
    np.testing.assert_allclose(got2, got, rtol=1e-12, atol=1e-13)
    # an empty list gives zeros; entries outside [0, nb) are skipped
    cnt0 = cnt.copy()
    cnt0[0, 0] = 0
    z = oracle.attention_lists_rows(q, k, v, idx, cnt0, rows)
    ids, _ = tile_membership(T, H, W)
    assert (z[ids == 0] == 0).all()
    cnt3 = np.full_like(cnt, maxcnt)
    idx3 = np.where(np.arange(maxcnt) % 2 == 0, -5, nb + 3).astype(np.int32)[None, None, :].repeat(nb, 1)
    for b, l in enumerate(lists):
        idx3[0, b, :len(l)] = l
    np.testing.assert_allclose(oracle.attention_lists_rows(q, k, v, idx3, cnt3, rows), got,
                               rtol=1e-12, atol=1e-13)


# --------------------------------- sampling with inclusion-probability weights --

def pooled_softmax(q, k, T, H, W, d):
    """Block-mean logits softmax, from tile slices and scipy: [nb][nb] for head 0."""
    ids, _ = tile_membership(T, H, W)
    nb = ids.max() + 1
    qf, kf = f64(q)[0].reshape(-1, d), f64(k)[0].reshape(-1, d)
    qm = np.stack([qf[ids == b].mean(0) for b in range(nb)])
    km = np.stack([kf[ids == b].mean(0) for b in range(nb)])
    return scipy.special.softmax(qm @ km.T / math.sqrt(d), axis=1)


def test_sip_extremes_reduce_to_dense_and_per_tile():
    T, H, W, d = 2, 16, 24, 16
    q, k, v = ti.random_qkv(T, H, W, 1, d, seed=31)
    nb = oracle.grid_blocks(T, H, W)[2]
    u = np.random.default_rng(1).random((1, nb, nb))
    rows = np.arange(T * H * W)
    idx, cnt, lw = oracle.sip_lists(q, k, u, 1e12)  # every inclusion probability 1
    assert (cnt == nb).all() and (lw == 0).all()
    got = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=lw)
    ref = sdpa(f64(q).reshape(1, -1, d), f64(k).reshape(1, -1, d), f64(v).reshape(1, -1, d))[0]
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    idx, cnt, lw = oracle.sip_lists(q, k, u, 0.0)  # only the own block
    assert (cnt == 1).all() and (idx[0, :, 0] == np.arange(nb)).all()


def test_sip_inclusion_follows_pooled_importance():
    T, H, W, d = 2, 16, 24, 16
    q, k, _ = ti.random_qkv(T, H, W, 1, d, seed=32, scale=3.0)
    nb = oracle.grid_blocks(T, H, W)[2]
    m = 2.5
    idx, cnt, lw = oracle.sip_lists(q, k, np.zeros((1, nb, nb)), m)  # u = 0 keeps every pi > 0
    assert (cnt == nb).all()
    p = pooled_softmax(q, k, T, H, W, d)
    pi = np.exp(-lw[0])
    want = np.minimum(1.0, m * p)
    np.fill_diagonal(want, 1.0)
    np.testing.assert_allclose(pi, want, rtol=1e-10)
    # a block is kept when its uniform falls below its inclusion probability
    b, c = 0, int(np.argmin(want[0] + np.eye(nb)[0]))
    assert want[b, c] < 1
    u = np.full((1, nb, nb), 0.999999)
    u[0, b, c] = want[b, c] * (1 + 1e-9)
    i2, c2, _ = oracle.sip_lists(q, k, u, m)
    assert c not in i2[0, b, :c2[0, b]].tolist()
    u[0, b, c] = want[b, c] * (1 - 1e-9)
    i3, c3, _ = oracle.sip_lists(q, k, u, m)
    assert c in i3[0, b, :c3[0, b]].tolist()


def test_sip_estimate_is_unbiased():
    # sum over kept blocks of exp(lw) S_K estimates sum over all blocks of S_K
    T, H, W, d = 2, 16, 16, 16
    q, k, v = ti.random_qkv(T, H, W, 1, d, seed=33, scale=2.0)
    nb = oracle.grid_blocks(T, H, W)[2]
    ids, _ = tile_membership(T, H, W)
    qf, kf = f64(q)[0].reshape(-1, d), f64(k)[0].reshape(-1, d)
    i = 5  # a query token of block 0
    s = kf @ qf[i] / math.sqrt(d)
    S = np.array([np.exp(s[ids == b] - s.max()).sum() for b in range(nb)])
    rng = np.random.default_rng(2)
    R = 3000
    est = np.empty(R)
    for r in range(R):
        idx, cnt, lw = oracle.sip_lists(q, k, rng.random((1, nb, nb)), 2.0)
        kept = idx[0, 0, :cnt[0, 0]]
        est[r] = (np.exp(lw[0, 0, :cnt[0, 0]]) * S[kept]).sum()
    se = est.std() / math.sqrt(R)
    assert se > 0
    assert abs(est.mean() - S.sum()) < 4 * se


def test_weighted_list_attention_identities():
    T, H, W, d = 2, 12, 16, 8
    q, k, v = ti.random_qkv(T, H, W, 1, d, seed=34)
    nb = oracle.grid_blocks(T, H, W)[2]
    rows = np.arange(T * H * W)
    idx = np.full((1, nb, 3), -1, dtype=np.int32)
    cnt = np.full((1, nb), 2, dtype=np.int32)
    for b in range(nb):
        idx[0, b, :2] = [b, (b + 1) % nb]
    # a log-weight of ln 2 on one entry counts that block twice
    lw = np.zeros((1, nb, 3))
    lw[0, :, 1] = math.log(2.0)
    got = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=lw)
    dup = idx.copy()
    dup[0, :, 2] = dup[0, :, 1]
    ref = oracle.attention_lists_rows(q, k, v, dup, np.full((1, nb), 3, dtype=np.int32), rows)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # a constant log-weight changes nothing
    const = oracle.attention_lists_rows(q, k, v, idx, cnt, rows, lw=np.full((1, nb, 3), 0.7))
    plain = oracle.attention_lists_rows(q, k, v, idx, cnt, rows)
    np.testing.assert_allclose(const, plain, rtol=1e-12, atol=1e-13)
