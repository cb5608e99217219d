"""The probe entry point that allocates nothing (tra_probe_static, its scratch a
static device array) against tra_probe, through the C ABI: bit-equal radii and
normalised entropies on two calls in a row, the second on a smaller input (the
array keeps the first call's contents), and the size limit."""
import numpy as np
import pytest

import tra_inputs as ti

torch = pytest.importorskip("torch")
import content_adaptive_sparse_amd as tra  # noqa: E402

pytestmark = pytest.mark.gpu


def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def probe_both(shape, r_min, r_max, seed):
    heads, T, H, W, d = shape
    q, k, _ = ti.make_inputs(T, H, W, heads, d, seed=seed, family=51)
    qd, kd = dev16(q), dev16(k)
    nb = tra.tra_grid(T, H, W)[2]
    out = []
    for fn in (tra.tra_probe_static, tra.tra_probe):
        r = torch.full((heads, nb), -9, dtype=torch.int32, device="cuda")
        hn = torch.full((heads, nb), float("nan"), dtype=torch.float32, device="cuda")
        fn(qd, kd, T, H, W, heads, d, 64, r_min, r_max, r, hn)
        torch.cuda.synchronize()
        out.append((r.cpu().numpy(), hn.cpu().numpy()))
    return out


def test_static_probe_matches_probe_on_two_calls():
    # first call larger than the second: the second must not see the first's
    # leftovers in the shared array
    for shape, (r_min, r_max), seed in (((3, 6, 30, 52, 128), (1, 8), 1),
                                         ((1, 2, 13, 9, 64), (0, 2), 2)):
        print(f"[case] tra_probe_static {shape} r=[{r_min},{r_max}]", flush=True)
        (r_s, hn_s), (r_p, hn_p) = probe_both(shape, r_min, r_max, seed)
        assert np.array_equal(r_s, r_p), f"{shape}: radii differ from tra_probe"
        assert np.array_equal(hn_s.view(np.uint32), hn_p.view(np.uint32)), f"{shape}: h_norm differs"
        assert (r_s >= r_min).all() and (r_s <= r_max).all()


def test_static_probe_size_limit():
    limit = tra.tra_static_scratch_bytes()
    # 64 heads of the HunyuanVideo-shaped grid: 2 x 64 x 1980 x 128 x 4 bytes of block means
    T, H, W, heads, d = 33, 45, 80, 64, 128
    assert tra.tra_workspace_bytes(T, H, W, heads, d, 64, 4) > limit
    x = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(tra.TraError) as e:
        tra.tra_probe_static(x, x, T, H, W, heads, d, 64, 1, 4, r)
    assert e.value.status == -5
