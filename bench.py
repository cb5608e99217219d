"""Benchmark of the entropy-radius block-sparse attention layer on one MI355X.

One step = one whole layer, ``tra_attention`` (probe -> radii -> key-block
lists -> block-sparse attention) over all heads, inputs resident in HBM.
Default workload: the Wan2.1-1.3B 480x832 81-frame layer (T=21, H=30, W=52,
12 heads, head_dim 128, bf16, 64-token 8x8 tiles, radii 1..8).

Prints one JSON line (last line of stdout) with ms/layer, the attention
kernel's achieved TFLOP/s on computed blocks against the dense bf16/fp16
matrix-core peak, the dense-mode time, an injected-radius density sweep and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/layer + effective TFLOP/s (fraction of bf16 MFMA peak) vs dense, Wan-1.3B shape"
PEAK_TFLOPS = 2500.0        # MI355X dense bf16 / fp16 matrix-core peak
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
INF = 2147483647
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tra_attn_traffic.json")
# the attention kernel and the walk plan it follows (pairing, walks, order):
# the counters in TRAFFIC_FILE hold for this pair of sources
ATTN_SRC = [os.path.join(ROOT, "content_adaptive_sparse_amd", "csrc", f)
            for f in ("tra_attn.hip", "tra_mask.hip")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def attn_source_hash():
    """sha256[:16] of the attention kernel and walk-plan sources with comments
    and white space removed: an edited comment keeps the counters valid, any
    change of code voids them."""
    h = hashlib.sha256()
    for path in ATTN_SRC:
        with open(path, encoding="utf-8") as f:
            code = _COMMENTS.sub(" ", f.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_key):
    """HBM bytes per attention launch from rocprofv3 counters, if they were
    taken on the current kernel source for this workload; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("attn_source_sha") != attn_source_hash() or rec.get("workload") != workload_key:
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(q, k, v, c, budget_s):
    """fp64 oracle on a bounded sample: full probe and block lists, then
    attention rows until about budget_s seconds; extrapolated to one layer."""
    import oracle
    t0 = time.perf_counter()
    hn, r = oracle.probe(q, k, c.r_min, c.r_max)
    oracle.block_lists(r, c.T, c.H, c.W, maxcnt=oracle.grid_blocks(c.T, c.H, c.W)[2])
    t_fixed = time.perf_counter() - t0
    total_rows = c.heads * c.N
    rng = np.random.default_rng(0)
    rows_done, t_rows, batch = 0, 0.0, 256
    while t_rows < budget_s and rows_done < total_rows:
        rows = rng.choice(total_rows, size=min(batch, total_rows), replace=False)
        t1 = time.perf_counter()
        oracle.attention_rows(q, k, v, r, rows)
        dt = time.perf_counter() - t1
        t_rows += dt
        rows_done += rows.size
        batch = int(min(max(batch, rows.size * max(budget_s - t_rows, 0.0) / max(dt, 1e-3)), 65536)) or 256
    ms_layer = 1e3 * (t_fixed + t_rows * total_rows / rows_done)
    return {
        "value": round(ms_layer, 1),
        "unit": "ms/layer",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"full fp64 probe + block lists ({t_fixed:.1f} s), then {rows_done} of "
                   f"{total_rows} query rows of masked attention on the same radii "
                   f"({t_rows:.1f} s), attention time extrapolated linearly to all rows"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the chip raises its clock over the first ~25 ms of work after an idle gap
    # (attention launches 3.3 ms at first, 2.55-2.6 ms once warm): 20 layers
    # (about 55 ms) reach the steady state
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wan13b_81f",
                    help="workload slug (tra_inputs.WORKLOADS): tiny, wan13b_81f, wan13b_241f, "
                         "wan14b_81f, hunyuan_129f")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU oracle sample budget (0 skips it)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--only-layer", action="store_true",
                    help="time the layer only (for profiler runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference for hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards "
              "by head with no communication, so there is no multi-GPU path to time.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import content_adaptive_sparse_amd as tra
    import tra_inputs as ti

    wid = {w.slug: i for i, w in ti.WORKLOADS.items()}.get(args.workload)
    if wid is None:
        print(f"unknown workload {args.workload!r}", file=sys.stderr)
        sys.exit(2)
    c = ti.WORKLOADS[wid]
    T, H, W, heads, d = c.T, c.H, c.W, c.heads, c.d
    nby, nbx, nb = tra.tra_grid(T, H, W)
    log(f"[bench] workload {c.name}; generating inputs", )
    q, k, v = ti.make_workload_inputs(wid)

    def dev(x):
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)

    qd, kd, vd = dev(q), dev(k), dev(v)
    out = torch.empty(heads, T, H, W, d, dtype=torch.float32, device="cuda")
    flops_pair = 4 * 64 * 64 * d
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        del src, dst

    def layer(r_min, r_max):
        tra.tra_attention(qd, kd, vd, T, H, W, heads, d, 64, r_min, r_max, out)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return e0.elapsed_time(e1) / steps, wall

    def profiled(fn, steps):
        torch.cuda.synchronize()
        tra.tra_profile_begin()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res = tra.tra_profile_end()
        return {kk: (ms / n if n else 0.0) for kk, (ms, n) in res.items()}

    # ---- the layer (timed region: exactly --steps calls) ----
    ms_layer, ms_wall = timed(lambda: layer(c.r_min, c.r_max), args.steps, args.warmup)
    log(f"[bench] layer {ms_layer:.3f} ms (wall {ms_wall:.3f})")
    if args.only_layer:
        ms_dense, _ = timed(lambda: layer(INF, INF), args.steps, args.warmup)
        log(f"[bench] dense layer {ms_dense:.3f} ms")
        return

    # per-step spread of the layer time (a separate pass: one event between
    # consecutive layers on the launch stream)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        layer(c.r_min, c.r_max)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    step_median, step_min = float(np.median(per_step)), float(np.min(per_step))
    log(f"[bench] layer per step: median {step_median:.3f} ms, min {step_min:.3f} ms")

    # realised radii / lists of the probe (same kernels as inside the layer)
    radius = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    tra.tra_probe(qd, kd, T, H, W, heads, d, 64, c.r_min, c.r_max, radius)
    maxcnt = tra.tra_maxcnt(T, H, W, 64, c.r_max)
    idx = torch.empty(heads, nb, maxcnt, dtype=torch.int32, device="cuda")
    cnt = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
    tra.tra_mask(radius, T, H, W, heads, 64, c.r_max, idx, cnt)
    torch.cuda.synchronize()
    pairs = int(cnt.sum().item())
    density = pairs / (heads * nb * nb)
    rhist = np.bincount(radius.cpu().numpy().ravel(), minlength=c.r_max + 1).tolist()
    del idx

    # ---- the attention kernel alone: `reps` back-to-back launches along the
    # probe radii's walk plan (built from the radii as the layer builds it)
    # between one pair of HIP events on the launch stream (no per-kernel
    # brackets); the same for the dense mode ----
    reps = max(10, args.steps)

    def radius_plan(rd, rmax):
        mc = tra.tra_maxcnt(T, H, W, 64, rmax)
        pl = torch.empty(tra.tra_plan_bytes(T, H, W, heads, 64, mc), dtype=torch.uint8,
                         device="cuda")
        tra.tra_plan_radius(rd, T, H, W, heads, 64, rmax, pl)
        return pl, mc

    # ten untimed launches before each timed run: after the host work between
    # the benchmark's phases the chip's clock ramps up again over the first
    # 25-30 ms of work
    plan, _ = radius_plan(radius, c.r_max)
    tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan, maxcnt, 10, out)
    t_attn = tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan, maxcnt, reps, out)
    tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, None, 0, 4, out)
    t_dense_attn = tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, None, 0, reps, out)
    del plan
    idx = torch.empty(heads, nb, maxcnt, dtype=torch.int32, device="cuda")
    tra.tra_mask(radius, T, H, W, heads, 64, c.r_max, idx, cnt)
    achieved = flops_pair * pairs / (t_attn * 1e-3) / 1e12
    dense_tflops = flops_pair * heads * nb * nb / (t_dense_attn * 1e-3) / 1e12
    # the same launch counted three ways: per computed 64 x 64 block pair (the
    # headline), per matrix-core product actually issued (a wave whose 32
    # queries are all padding issues none), and per real (query, key) token pair
    cn_h = cnt.cpu().numpy().astype(np.int64)
    ix_h = idx.cpu().numpy()
    qn = np.array([min(8, H - 8 * ((b // nbx) % nby)) * min(8, W - 8 * (b % nbx)) for b in range(nb)])
    waves = (qn + 31) // 32
    mfma_flops = 4 * 32 * 64 * d * int((cn_h * waves[None, :]).sum())
    kreal = np.zeros(heads * nb, dtype=np.int64)
    for h in range(heads):
        for b in range(nb):
            kreal[h * nb + b] = qn[ix_h[h, b, :cn_h[h, b]]].sum()
    real_flops = 4 * d * int((kreal.reshape(heads, nb) * qn[None, :]).sum())
    del idx, ix_h
    log(f"[bench] attention kernel {t_attn:.4f} ms ({achieved:.1f} TFLOP/s on computed blocks), "
        f"dense {t_dense_attn:.4f} ms ({dense_tflops:.1f} TFLOP/s)")

    # diagnostic only: every kernel of the layer bracketed by its own event pair
    # (the brackets add their own gaps, so these sum to more than the layer)
    kern = profiled(lambda: layer(c.r_min, c.r_max), max(5, args.steps // 2))
    log(f"[bench] bracketed kernels (ms): {kern}; density {density:.4f}")

    # ---- dense mode of the same kernel ----
    ms_dense, _ = timed(lambda: layer(INF, INF), max(3, args.steps // 2), 2)
    log(f"[bench] dense layer {ms_dense:.3f} ms")

    # Attention kernel alone along other walks: one untimed launch (a kernel's
    # first launch in the process also loads its code), then the best of three
    # runs of 10 back-to-back launches (the first runs on fresh scratch memory
    # measured up to 15% slower).
    def attn_time(ix, cn, mc, lw=None):
        tra.tra_time_attn(qd, kd, vd, T, H, W, heads, d, 64, ix, cn, lw, mc, 1, out)
        return min(tra.tra_time_attn(qd, kd, vd, T, H, W, heads, d, 64, ix, cn, lw, mc, 10, out)
                   for _ in range(3))

    def attn_time_radii(rd, rmax):
        pl, mc = radius_plan(rd, rmax)
        tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, pl, mc, 1, out)
        return min(tra.tra_time_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, pl, mc, 10, out)
                   for _ in range(3))

    # ---- injected-radius density sweep (attention kernel only) ----
    sweep = []
    if not args.no_sweep:
        rng = np.random.default_rng(0)
        cases = [("r=1", np.ones((heads, nb))), ("r=2", np.full((heads, nb), 2)),
                 ("r in {1,2}", rng.integers(1, 3, size=(heads, nb))),
                 ("r in {2,3}", rng.integers(2, 4, size=(heads, nb)))]
        for name, rr in cases:
            rmax = int(rr.max())
            rd = torch.from_numpy(rr.astype(np.int32)).cuda()
            mc = tra.tra_maxcnt(T, H, W, 64, rmax)
            ix = torch.empty(heads, nb, mc, dtype=torch.int32, device="cuda")
            cn = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
            tra.tra_mask(rd, T, H, W, heads, 64, rmax, ix, cn)
            torch.cuda.synchronize()
            p = int(cn.sum().item())
            ta = attn_time_radii(rd, rmax)
            sweep.append({"radii": name, "density": round(p / (heads * nb * nb), 4),
                          "attn_ms": round(ta, 4),
                          "tflops": round(flops_pair * p / (ta * 1e-3) / 1e12, 1),
                          "speedup_vs_dense_attn": round(t_dense_attn / ta, 2)})
            log(f"[bench] sweep {sweep[-1]}")
            del ix, cn

    # ---- cross-step reuse: probe and walk plan once (the warm-up step); every
    # later step packs k, v and runs the attention along the stored plan ----
    reuse, routing, route_lists = None, None, None
    if not args.no_sweep:
        plan, _ = radius_plan(radius, c.r_max)
        step = lambda: tra.tra_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan, maxcnt, out)
        ms_reuse, _ = timed(step, max(5, args.steps // 2), 2)
        reuse = {"ms_per_step": round(ms_reuse, 4),
                 "speedup_vs_dense_layer": round(ms_dense / ms_reuse, 3),
                 "plan_bytes": int(plan.numel())}
        log(f"[bench] cross-step reuse {reuse}")
        del plan

        # ---- binary routing: the 20% of blocks per head with the highest
        # pooled-probe entropy attend densely, the rest with radius 1 ----
        hn = torch.empty(heads, nb, dtype=torch.float32, device="cuda")
        rtmp = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
        tra.tra_probe(qd, kd, T, H, W, heads, d, 64, c.r_min, c.r_max, rtmp, hn)
        hnn = hn.cpu().numpy()
        cut = np.quantile(hnn, 0.8, axis=1, keepdims=True)
        rr = np.where(hnn >= cut, INF, 1).astype(np.int32)
        rd = torch.from_numpy(rr).cuda()
        ix = torch.empty(heads, nb, nb, dtype=torch.int32, device="cuda")
        cn = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
        tra.tra_mask(rd, T, H, W, heads, 64, INF, ix, cn)
        torch.cuda.synchronize()
        cnn = cn.cpu().numpy()
        p = int(cnn.sum())
        ta = attn_time(ix, cn, nb)
        routing = {"dense_blocks": round(float((rr == INF).mean()), 4), "local_radius": 1,
                   "density": round(p / (heads * nb * nb), 4),
                   "list_len_min_mean_max": [int(cnn.min()), round(float(cnn.mean()), 1), int(cnn.max())],
                   "attn_ms": round(ta, 4),
                   "tflops": round(flops_pair * p / (ta * 1e-3) / 1e12, 1),
                   "speedup_vs_dense_attn": round(t_dense_attn / ta, 2)}
        log(f"[bench] binary routing {routing}")
        route_lists = (ix, cn)
        del rd

    # ---- token-level radius policy: the warm-up (dense attention with every
    # token's entropy and base radius in the same pass, then the voting mask and
    # the walk plan), then steps reusing those lists ----
    token = None
    if not args.no_sweep:
        tau, gamma, mv = 1.0, 0.5, 1
        N = T * H * W
        ent = torch.empty(heads, T, H, W, dtype=torch.float32, device="cuda")
        r0 = torch.empty_like(ent)
        ix = torch.empty(heads, nb, nb, dtype=torch.int32, device="cuda")
        cn = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
        plan = torch.empty(tra.tra_plan_bytes(T, H, W, heads, 64, nb), dtype=torch.uint8, device="cuda")

        def warmup_step():
            tra.tra_token_warmup(qd, kd, vd, T, H, W, heads, d, 64, tau, gamma, out, ent, r0)
            tra.tra_token_mask(r0, T, H, W, heads, 64, gamma, mv, ix, cn)
            tra.tra_plan(ix, cn, nb, T, H, W, heads, 64, plan)

        ms_warm_attn, _ = timed(lambda: tra.tra_token_warmup(qd, kd, vd, T, H, W, heads, d, 64, tau,
                                                             gamma, out, ent, r0), 5, 1)
        ms_warm, _ = timed(warmup_step, 5, 1)
        kp = profiled(lambda: tra.tra_token_probe(qd, kd, T, H, W, heads, d, 64, tau, gamma, ent, r0), 3)
        torch.cuda.synchronize()
        p = int(cn.sum().item())
        ta = attn_time(ix, cn, nb)
        ms_step, _ = timed(lambda: tra.tra_attn_plan(qd, kd, vd, T, H, W, heads, d, 64, plan, nb, out),
                           max(5, args.steps // 2), 2)
        ms_one_call, _ = timed(lambda: tra.tra_token_attention(qd, kd, vd, T, H, W, heads, d, 64, tau,
                                                               gamma, mv, out), 3, 1)
        token = {"tau": tau, "gamma": gamma, "min_votes": mv,
                 "entropy_h_mean": round(float(ent.mean().item()), 3), "ln_N": round(math.log(N), 3),
                 "density": round(p / (heads * nb * nb), 4),
                 "warmup_step_ms": round(ms_warm, 4),
                 "warmup_dense_attn_with_entropy_ms": round(ms_warm_attn, 4),
                 "warmup_step_vs_dense_layer": round(ms_warm / ms_dense, 3),
                 "separate_entropy_pass_ms": round(kp["token_entropy"], 4),
                 "attn_ms": round(ta, 4),
                 "attn_tflops": round(flops_pair * p / (ta * 1e-3) / 1e12, 1),
                 "reuse_step_ms": round(ms_step, 4),
                 "reuse_speedup_vs_dense_layer": round(ms_dense / ms_step, 3),
                 "one_call_ms": round(ms_one_call, 4)}
        log(f"[bench] token policy {token}")
        del ix, cn, plan, ent, r0

    # ---- sampling with inclusion-probability weights (seeded device uniforms),
    # and how far each scheme's output is from dense attention ----
    sip, quality = [], None
    if not args.no_sweep:
        out_dense = torch.empty_like(out)
        tra.tra_attention(qd, kd, vd, T, H, W, heads, d, 64, INF, INF, out_dense)

        def l1_vs_dense():
            torch.cuda.synchronize()
            return round(float((out - out_dense).abs().sum() / out_dense.abs().sum()), 5)

        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        u = torch.rand(heads, nb, nb, device="cuda", generator=gen)
        ix = torch.empty(heads, nb, nb, dtype=torch.int32, device="cuda")
        cn = torch.empty(heads, nb, dtype=torch.int32, device="cuda")
        lw = torch.empty(heads, nb, nb, dtype=torch.float32, device="cuda")
        for m in (64.0, 256.0, 1024.0):
            ks = profiled(lambda: tra.tra_sip_mask(qd, kd, u, T, H, W, heads, d, 64, m, ix, cn, lw), 3)
            torch.cuda.synchronize()
            p = int(cn.sum().item())
            ta = attn_time(ix, cn, nb, lw)
            tra.tra_attn_weighted(qd, kd, vd, T, H, W, heads, d, 64, ix, cn, lw, nb, out)
            sip.append({"m": m, "density": round(p / (heads * nb * nb), 4),
                        "sip_mask_ms": round(ks["sip"] + ks["entropy"] + ks["pack_pool"], 4),
                        "attn_ms": round(ta, 4),
                        "tflops": round(flops_pair * p / (ta * 1e-3) / 1e12, 1),
                        "l1_vs_dense": l1_vs_dense()})
            log(f"[bench] sip {sip[-1]}")
        del ix, cn, lw, u
        quality = {}
        layer(c.r_min, c.r_max)
        quality["probe_radii"] = {"density": round(density, 4), "l1_vs_dense": l1_vs_dense()}
        if token is not None:
            tra.tra_token_attention(qd, kd, vd, T, H, W, heads, d, 64, token["tau"], token["gamma"],
                                    token["min_votes"], out)
            quality["token_policy"] = {"density": token["density"], "l1_vs_dense": l1_vs_dense()}
        if routing is not None:
            tra.tra_attn(qd, kd, vd, T, H, W, heads, d, 64, route_lists[0], route_lists[1], nb, out)
            quality["binary_routing"] = {"density": routing["density"], "l1_vs_dense": l1_vs_dense()}
        quality["sip"] = [{"density": e["density"], "l1_vs_dense": e["l1_vs_dense"]} for e in sip]
        log(f"[bench] output error vs dense attention {quality}")
        del out_dense, route_lists

    # HBM bandwidth of the probe/pack kernel (algorithmic bytes: read q, k, v,
    # write the packed k and v^T tiles and the pooled means)
    pack_bytes = 3 * heads * c.N * d * 2 + 2 * heads * nb * 64 * d * 2 + 2 * heads * nb * d * 4
    pack_gbs = pack_bytes / (kern["pack_pool"] * 1e-3) / 1e9
    mask_bytes = 4 * (heads * nb + pairs)
    mask_gbs = mask_bytes / (kern["mask"] * 1e-3) / 1e9 if kern["mask"] > 0 else None

    workload_key = c.slug
    traffic = measured_traffic(workload_key)
    res = {
        "metric": METRIC,
        "value": round(ms_layer, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_layer, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": c.name,
            "T": T, "H": H, "W": W, "heads": heads, "head_dim": d, "block": 64,
            "r_min": c.r_min, "r_max": c.r_max, "batch": 1,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "details": {
            "effective_tflops_attn": round(achieved, 1),
            "frac_of_bf16_peak": round(achieved / PEAK_TFLOPS, 4),
            "effective_tflops_layer": round(flops_pair * pairs / (ms_layer * 1e-3) / 1e12, 1),
            "block_density": round(density, 4),
            "computed_block_pairs": pairs,
            "radius_histogram": rhist,
            "attn_ms": round(t_attn, 4),
            "attn_timing": (f"mean of {reps} back-to-back attention launches between one HIP event "
                            "pair on the launch stream, after ten untimed launches, along the walk plan the "
                            "layer builds from the radii (tra_plan_radius, tra_time_attn_plan)"),
            "mfma_executed_tflops_attn": round(mfma_flops / (t_attn * 1e-3) / 1e12, 1),
            "real_token_tflops_attn": round(real_flops / (t_attn * 1e-3) / 1e12, 1),
            "flops_per_launch": {"computed_block_pairs": flops_pair * pairs,
                                 "mfma_executed": mfma_flops, "real_token_pairs": real_flops},
            "kernel_ms_bracketed_diagnostic": {kk: round(vv, 4) for kk, vv in kern.items() if vv},
            "dense_ms_per_layer": round(ms_dense, 4),
            "dense_attn_ms": round(t_dense_attn, 4),
            "dense_attn_tflops": round(dense_tflops, 1),
            "speedup_vs_dense_layer": round(ms_dense / ms_layer, 3),
            "pack_pool_gbs": round(pack_gbs, 1),
            "mask_gbs": None if mask_gbs is None else round(mask_gbs, 2),
            "density_sweep": sweep,
            "cross_step_reuse": reuse,
            "binary_routing": routing,
            "token_policy": token,
            "sip_sweep": sip,
            "l1_vs_dense_by_scheme": quality,
            "wall_ms_per_step": round(ms_wall, 4),
            "layer_ms_median": round(step_median, 4),
            "layer_ms_min": round(step_min, 4),
            "pv_dtype": "fp16",
        },
    }
    if args.cpu_seconds > 0:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(q, k, v, c, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
