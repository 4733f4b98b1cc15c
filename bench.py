#!/usr/bin/env python3
"""Benchmark of the warp-decode MoE layer on one MI355X.

One step = one pass of the whole layer (moe_decode_gate_up then
moe_decode_down) over one batch: B=32 tokens through one MoE layer of
H=2048, E=128 experts, top-8 routing, I=768, MXFP8 weights, with fresh
uniform routing and activations every step.  Inputs are resident in HBM
before the timed region starts.

Metric: effective HBM GB/s = algorithmic bytes / time, where the algorithmic
bytes of one step are the distinct routed experts' weights and scales plus
activations, routing, the intermediate's write and read, and the output
(layer_bytes below).  Also reported: microseconds per layer, the fraction of a
copy-kernel peak measured in the same process (the efficiency figure of the
blog post's "Hardware efficiency" section), a B sweep, the dominant kernel's
roofline position, the conventional expert-centric path timed on the same
batches (the blog post's "Stage elimination" A/B), the top-k router step in
front of the layer (fused into gate/up and as its own kernel), and the CPU
oracle timed on the host as a baseline.

Weights: one layer is generated on the host (seed 0) and uploaded; the other
`--copies` - 1 layers (47 more for the 48-layer step, 7 for the wide shape)
are made on the device from it, each with every weight's sign flipped by its
own seeded random mask, so every layer holds distinct weights of the same
distribution at its own addresses.  Step i uses layer i mod copies, so
consecutive steps never read the same addresses and the 256 MB last-level
cache (MALL) cannot serve a step from the previous one.

The timed loops are captured into HIP graphs and replayed, as a decode server
would run a step; the timed region starts after the inputs are resident.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE decode layer effective HBM GB/s (% of copy peak) + µs/layer, B=1..32"
HBM_PEAK_GBPS = 8000.0   # MI355X published HBM3E bandwidth
# Timing: after the host synchronises, the GPU's clocks take ~20 ms of work to
# settle (B=32 per-step time over loops of 50..800 steps: 111.7, 107.3, 105.9,
# 105.7, 105.7 us), so every timed graph is first replayed untimed for >= 20 ms
# and then timed over >= 5 back-to-back replays (median reported, p10/p90 beside).
SETTLE_S = 0.02
TIMED_REPLAYS = 5
MAX_TIMED_REPLAYS = 50


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PEAK_SIZES_MB = (256, 512, 1024, 4096)


def measure_peaks(dev, sizes_mb=PEAK_SIZES_MB):
    """Copy and read probe rates at each transfer size, graph-replayed (no
    launch gaps between passes), each pass on other buffers than the previous
    one; returns (best copy GB/s counting read + written bytes, best read GB/s,
    the per-size table)."""
    import torch
    import moe_gate_up_amd as mg

    span = 2 * (max(sizes_mb) << 20)
    buf = torch.empty(max(span, 6 << 30), dtype=torch.uint8, device=dev)
    buf.fill_(7)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(run, reps):
        for i in range(2):
            run(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                run(i)
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) / 1e3 / reps)
        del g
        return best

    table = []
    for mb in sizes_mb:
        n = mb << 20
        slots = max(1, min(6, buf.numel() // (2 * n)))
        pairs = [(buf[2 * i * n:(2 * i + 1) * n], buf[(2 * i + 1) * n:(2 * i + 2) * n]) for i in range(slots)]
        reps = max(2, min(32, (8 << 30) // (2 * n)))
        tc = timed(lambda i: mg.moe_decode_copy_peak(pairs[i % slots][0], pairs[i % slots][1]), reps)
        tr = timed(lambda i: mg.moe_decode_read_peak(pairs[i % slots][(i // slots) % 2], sink), reps)
        table.append({"MB": mb, "copy_GBps": round(2 * n / tc / 1e9, 1), "read_GBps": round(n / tr / 1e9, 1)})
    del buf, sink
    torch.cuda.empty_cache()
    return max(p["copy_GBps"] for p in table), max(p["read_GBps"] for p in table), table


def layer_bytes(ids: np.ndarray, H: int, I: int, k: int) -> dict:
    """Algorithmic bytes of one layer pass for the given routing ids [B,k].

    Per distinct routed expert: gate, up and down rows (3*I*H E4M3 bytes) plus
    their E8M0 scales (3*I*H/32).  Per token: x read (2H), y write (2H).  Per
    slot: h written then read (2 * 2I), id read by both kernels (8), router
    weight (4)."""
    B = ids.shape[0]
    D = len(np.unique(ids))
    w = D * (3 * I * H + 3 * I * H // 32)
    gate_up = D * (2 * I * H + 2 * I * H // 32) + 2 * B * H + 2 * B * k * I + 4 * B * k
    down = D * (I * H + I * H // 32) + 2 * B * k * I + 8 * B * k + 2 * B * H
    return dict(distinct=D, weights=w, total=gate_up + down, gate_up=gate_up, down=down)


_GATE_UP_KERNELS = {1: "per-slot", 2: "vector-unit grouped", 3: "matrix-core grouped"}
_DOWN_KERNELS = {1: "per-token", 2: "vector-unit grouped", 3: "matrix-core grouped"}


def kernel_choice(B: int, H: int, I: int, E: int, k: int) -> str:
    """The built-in table's kernels for this shape (what the plain calls run)."""
    import moe_gate_up_amd as mg
    vg = mg.moe_decode_gate_up_plan(B, H, I, E, k)[0]
    vd = mg.moe_decode_down_plan(B, H, I, E, k)[0]
    return f"gate_up {_GATE_UP_KERNELS.get(vg, vg)}, down {_DOWN_KERNELS.get(vd, vd)}"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "moe_gate_up_amd", "csrc")
    for f in sorted(os.listdir(d)):   # every kernel source and header of the library
        if f.endswith((".hpp", ".hip")):
            h.update(f.encode() + b"\0" + open(os.path.join(d, f), "rb").read())
    # and the compiler flags they are built with
    h.update(b"build.py\0" + open(os.path.join(ROOT, "moe_gate_up_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, name: str = None, workload: dict = None):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
    reads for a copy kernel of known size) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources -- and, where given, on
    the kernel `name` and the `workload` (shape and routing) asked about; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    if workload is not None and d.get("workload") != workload:
        return None
    k = d.get("kernels", {}).get(kernel)
    if k is None or (name is not None and not k.get("template_name", "").startswith(name)):
        return None
    return k.get("bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--copies", type=int, default=8, help="device copies of the layer weights, cycled per step")
    ap.add_argument("--routings", type=int, default=64, help="pre-generated routings, cycled per step")
    ap.add_argument("--sweep", default="1,2,4,8,16,32", help="batch sizes for the sweep ('' to skip)")
    # per-step time settles after ~100 steps of a replay (50: +5.6 %, 100: +1.5 %,
    # 200: +0.2 % over 400-800 steps at B=32 on MI355X); 200 is within noise
    ap.add_argument("--sweep-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the routing-stress, 48-layer and wide-shape runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the all-threads oracle sample (one more pass runs on one thread)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the layer would shard I across GPUs with one all-reduce of y; not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_gate_up_amd as mg
    import moe_inputs as mi

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mg.lib()   # fail loudly if the HIP library is missing

    S = mi.SHAPES["S1"]
    H, I, E, k = S["H"], S["I"], S["E"], S["k"]
    t0 = time.time()
    L = mi.make_layer(mi.layer_seed("batch_sweep"), H, I, E)
    log(f"generated layer in {time.time() - t0:.1f}s ({L.nbytes / 1e6:.1f} MB)")

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    host_w = (L.w_gate, L.s_gate, L.w_up, L.s_up, L.w_down, L.s_down)
    first = [up(a) for a in host_w]

    def distinct(ws, n):
        """Layer n: a copy of the layer at other addresses with every E4M3 weight's
        sign flipped by a seeded random mask (magnitudes and scale codes kept), so
        that every layer holds distinct weights of the same distribution.  The
        mask is drawn 16 MB at a time, so that no large temporary sits between
        the layers in device memory."""
        out = [t.clone() for t in ws]
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + n)
        for j in (0, 2, 4):   # w_gate, w_up, w_down (codes); the scale tensors stay as they are
            flat = out[j].view(-1)
            for o in range(0, flat.numel(), 1 << 24):
                part = flat[o:o + (1 << 24)]
                part.bitwise_xor_(torch.randint(0, 2, part.shape, generator=g, device=dev, dtype=torch.uint8) * 128)
        return out

    copies = [first] + [distinct(first, n) for n in range(1, args.copies)]
    torch.cuda.synchronize()
    log(f"{args.copies} distinct layers resident ({args.copies * L.nbytes / 1e9:.2f} GB)")

    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- copy peak
    # The copy kernel's rate depends on the transfer size (on MI355X it falls
    # by ~12 % from 512 MB to 4 GiB), so the peak is the best rate over a few
    # sizes; every size cycles through buffers far enough apart that no pass
    # finds its data in the 256 MB memory-side cache.
    copy_gbps, read_gbps, peak_by_size = measure_peaks(dev)
    log("copy / read probe by size: " + ", ".join(
        f"{p['MB']} MB {p['copy_GBps']:.0f}/{p['read_GBps']:.0f}" for p in peak_by_size))
    log(f"copy peak {copy_gbps:.0f} GB/s (read+write), read peak {read_gbps:.0f} GB/s")

    # ---------------------------------------------------------------- routed steps
    def make_batch(shape, B, n, kind, seed):
        H_, I_, E_, k_ = shape
        xs, ids_l, ws, info = [], [], [], []
        for r in range(n):
            xs.append(mi.make_x(seed, B, H_, it=r))
            ids, w = mi.make_routing(kind, seed, B, E_, k_, it=r)
            ids_l.append(ids)
            ws.append(w)
            info.append(layer_bytes(ids, H_, I_, k_))
        return (up(np.stack(xs)), up(np.stack(ids_l)), up(np.stack(ws)), info)

    def run_steps(wcopies, shape, B, steps, warmup, n_rout, kind="uniform", seed=None, layers=1, kernels=True,
                  path="warp"):
        """Time `steps` steps; a step is `layers` whole-layer passes (both kernels),
        layer l of a step reading weight copy l (cycled) with its own routing.
        Then each kernel alone in a back-to-back loop of steps*layers launches.

        Each loop is captured once into a HIP graph (torch.cuda.CUDAGraph) and the
        graph is replayed inside the timed region, so the figure is the GPU's time
        for the launches and not the Python launch overhead, which at small B
        exceeds the kernels' own duration.  Warm-up passes run eagerly first."""
        H_, I_, E_, k_ = shape
        seed = mi.routing_seed("batch_sweep", B) if seed is None else seed
        xs, idss, wss, info = make_batch(shape, B, n_rout, kind, seed)
        h = torch.empty((B, k_, I_), dtype=torch.int16, device=dev)
        y = torch.empty((B, H_), dtype=torch.int16, device=dev)

        def gate_up(i):
            wg, sg, wu, su, _, _ = wcopies[i % len(wcopies)]
            r = i % n_rout
            mg.moe_decode_gate_up(xs[r], idss[r], wg, sg, wu, su, h)

        def down(i):
            _, _, _, _, wd, sd = wcopies[i % len(wcopies)]
            r = i % n_rout
            mg.moe_decode_down(h, idss[r], wss[r], wd, sd, y)

        ws = None
        if path == "conventional":   # the expert-centric A/B path: seven launches through a workspace
            ws = torch.empty(mg.moe_decode_conventional_workspace(B, H_, I_, E_, k_), dtype=torch.uint8, device=dev)
        lgs = None
        if path in ("routed", "route_kernel"):
            # the router step in the timed loop: logits in (the draw behind the uniform
            # routing, so the same ids), ids and weights written on the device
            assert kind == "uniform"
            lgs = up(np.stack([mi.router_logits(seed, B, E_, it=r) for r in range(n_rout)]))
            rid = torch.empty((B, k_), dtype=torch.int32, device=dev)
            rw = torch.empty((B, k_), dtype=torch.float32, device=dev)

        def layer(i):
            wg, sg, wu, su, wd, sd = wcopies[i % len(wcopies)]
            r = i % n_rout
            if ws is not None:
                mg.moe_decode_conventional(xs[r], idss[r], wss[r], wg, sg, wu, su, wd, sd, y, ws)
            elif path == "routed":   # router step fused into gate/up, then down
                mg.moe_decode_gate_up_routed(xs[r], lgs[r], wg, sg, wu, su, h, rid, rw)
                mg.moe_decode_down(h, rid, rw, wd, sd, y)
            elif path == "vector":   # both kernels on the vector units (no matrix cores)
                mg.moe_decode_gate_up(xs[r], idss[r], wg, sg, wu, su, h, variant=mg.MOE_GATE_UP_EXPERT_GROUPED)
                mg.moe_decode_down(h, idss[r], wss[r], wd, sd, y, variant=mg.MOE_DOWN_EXPERT_GROUPED)
            elif path == "route_kernel":   # router kernel, then the two layer kernels
                mg.moe_decode_route(lgs[r], rid, rw)
                mg.moe_decode_gate_up(xs[r], rid, wg, sg, wu, su, h)
                mg.moe_decode_down(h, rid, rw, wd, sd, y)
            else:
                gate_up(i)
                down(i)

        def timed(fn, n):
            """Per-replay seconds of the graph of n launches of fn: the eager
            warm-up passes, untimed replays until the GPU has run >= SETTLE_S of
            this loop (clocks settle only after ~20 ms of work once the host has
            synchronised), then >= TIMED_REPLAYS back-to-back replays, each between
            two events on the launch stream, with one synchronisation before the
            first and after the last.  Returns (sorted per-replay seconds, wall
            seconds of the timed replays)."""
            for i in range(warmup * layers):
                fn(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    fn(warmup * layers + i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            first = max(a.elapsed_time(b) / 1e3, 1e-6)
            for _ in range(min(1000, int(SETTLE_S / first))):
                g.replay()
            reps = max(TIMED_REPLAYS, min(MAX_TIMED_REPLAYS, int(SETTLE_S / first)))
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            ev[0].record(stream)
            for r in range(reps):
                g.replay()
                ev[r + 1].record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - w0
            del g
            return sorted(ev[r].elapsed_time(ev[r + 1]) / 1e3 for r in range(reps)), wall

        def stats(ts):
            """median, p10, p90 of per-replay seconds"""
            q = np.quantile(np.asarray(ts), [0.5, 0.1, 0.9])
            return float(q[0]), float(q[1]), float(q[2])

        n = steps * layers
        ts, wall = timed(layer, n)
        t, t10, t90 = stats(ts)
        # sanity: outputs are finite (parity itself is checked by the test suite)
        assert torch.isfinite(y.view(torch.bfloat16).float()).all().item()
        pick = [info[(warmup * layers + i) % n_rout] for i in range(n)]
        byt = sum(d["total"] for d in pick)
        res = dict(B=B, seconds=t, wall_seconds=wall, replays=len(ts), bytes=byt, us_per_layer=t / n * 1e6,
                   us_per_layer_p10=t10 / n * 1e6, us_per_layer_p90=t90 / n * 1e6,
                   us_per_step=t / steps * 1e6, GBps=byt / t / 1e9,
                   distinct_experts=float(np.mean([d["distinct"] for d in info])))
        if path == "warp":
            res["kernels"] = kernel_choice(B, H_, I_, E_, k_)
        if kernels:
            t_gu = stats(timed(gate_up, n)[0])[0]
            t_dn = stats(timed(down, n)[0])[0]
            gub = sum(d["gate_up"] for d in pick)
            dnb = sum(d["down"] for d in pick)
            res.update(gate_up_us=t_gu / n * 1e6, down_us=t_dn / n * 1e6,
                       gate_up_GBps=gub / t_gu / 1e9, down_GBps=dnb / t_dn / 1e9,
                       gate_up_bytes_per_launch=gub / n, down_bytes_per_launch=dnb / n)
        return res

    def brief(r, keys=("B", "us_per_layer", "us_per_step", "GBps", "frac_of_copy_peak", "distinct_experts",
                       "gate_up_us", "down_us", "gate_up_GBps", "down_GBps", "routing", "layers",
                       "us_per_layer_p10", "us_per_layer_p90", "kernels")):
        return {kk: (round(r[kk], 4) if isinstance(r[kk], float) else r[kk]) for kk in keys if kk in r}

    S1 = (H, I, E, k)
    B = args.batch
    main_res = run_steps(copies, S1, B, args.steps, args.warmup, args.routings)
    kern = main_res
    log(f"B={B}: {main_res['us_per_layer']:.2f} us/layer, {main_res['GBps']:.0f} GB/s effective "
        f"({main_res['GBps'] / copy_gbps:.1%} of copy peak)")
    log(f"B={B} per kernel: gate_up {kern['gate_up_us']:.2f} us ({kern['gate_up_GBps']:.0f} GB/s), "
        f"down {kern['down_us']:.2f} us ({kern['down_GBps']:.0f} GB/s)")

    # the same workload with both kernels on the vector units only (expert-grouped
    # gate/up and down without matrix-core products)
    vec = run_steps(copies, S1, B, args.steps, args.warmup, args.routings, kernels=False, path="vector")
    log(f"B={B} on the vector units only: {vec['us_per_layer']:.2f} us/layer, {vec['GBps']:.0f} GB/s "
        f"({vec['GBps'] / copy_gbps:.1%} of copy peak)")

    sweep = []
    for b in [int(v) for v in args.sweep.split(",") if v.strip()]:
        r = run_steps(copies, S1, b, args.sweep_steps, 10, args.routings)
        r["frac_of_copy_peak"] = r["GBps"] / copy_gbps
        sweep.append(brief(r))
        log(f"sweep B={b}: {r['us_per_layer']:.2f} us/layer, {r['GBps']:.0f} GB/s ({r['frac_of_copy_peak']:.1%}); "
            f"gate_up {r['gate_up_us']:.2f} us, down {r['down_us']:.2f} us ({r['kernels']})")

    extra = {}
    if not args.no_configs:
        # routing stress at B=32: Zipf(1.1) popularity, adversarial (ids >= 3 apart), contiguous control
        c3 = []
        for kind in ("zipf", "adversarial", "contiguous"):
            r = run_steps(copies, S1, 32, args.sweep_steps, 10, args.routings, kind=kind,
                          seed=mi.routing_seed("routing_stress", 32, kind))
            r["frac_of_copy_peak"] = r["GBps"] / copy_gbps
            r["routing"] = kind
            c3.append(brief(r))
            log(f"routing {kind} B=32: {r['us_per_layer']:.2f} us/layer, {r['GBps']:.0f} GB/s "
                f"({r['frac_of_copy_peak']:.1%}), {r['distinct_experts']:.1f} distinct experts")
        extra["routing_stress_b32"] = c3

        # A/B: the conventional expert-centric path (route, pad, quantise, scatter, per-expert
        # buffers, combine: seven launches) on the same weights, routings and batches
        ab = []
        warp = {r["B"]: r for r in sweep}
        for b in (1, 8, 32):
            rw = warp.get(b) or brief(run_steps(copies, S1, b, args.sweep_steps, 10, args.routings, kernels=False))
            rc = run_steps(copies, S1, b, args.sweep_steps, 10, args.routings, kernels=False, path="conventional")
            ab.append({"B": b, "warp_decode_us_per_layer": round(rw["us_per_layer"], 3),
                       "conventional_us_per_layer": round(rc["us_per_layer"], 3),
                       "speedup": round(rc["us_per_layer"] / rw["us_per_layer"], 3)})
            log(f"conventional path B={b}: {rc['us_per_layer']:.2f} us/layer vs warp decode "
                f"{rw['us_per_layer']:.2f} us ({rc['us_per_layer'] / rw['us_per_layer']:.2f}x)")
        extra["conventional_ab"] = ab

        # the router step (top-8 of 128 logits, softmax over the kept 8) in front of the
        # layer: fused into gate/up vs its own kernel, against the layer with ids given
        ra = []
        for b in (1, 8, 32):
            rw = warp.get(b) or brief(run_steps(copies, S1, b, args.sweep_steps, 10, args.routings, kernels=False))
            rf = run_steps(copies, S1, b, args.sweep_steps, 10, args.routings, kernels=False, path="routed")
            rk = run_steps(copies, S1, b, args.sweep_steps, 10, args.routings, kernels=False, path="route_kernel")
            ra.append({"B": b, "ids_given_us_per_layer": round(rw["us_per_layer"], 3),
                       "router_fused_us_per_layer": round(rf["us_per_layer"], 3),
                       "router_kernel_us_per_layer": round(rk["us_per_layer"], 3)})
            log(f"router step B={b}: fused {rf['us_per_layer']:.2f} us/layer, own kernel "
                f"{rk['us_per_layer']:.2f}, ids given {rw['us_per_layer']:.2f}")
        extra["router_ab"] = ra

        # 48-layer decode step: 48 weight copies at distinct addresses, fresh routing per layer
        deep = [copies[i] if i < len(copies) else distinct(first, i) for i in range(48)]
        torch.cuda.synchronize()
        c4 = []
        for b in (1, 8, 32):
            r = run_steps(deep, S1, b, 10, 2, 96, seed=4000, layers=48, kernels=False)
            r["frac_of_copy_peak"] = r["GBps"] / copy_gbps
            r["layers"] = 48
            # the same step with each layer's routing made on the device from its N(0,1) logits
            rr = run_steps(deep, S1, b, 10, 2, 96, seed=4000, layers=48, kernels=False, path="routed")
            r["us_per_step_with_router"] = rr["us_per_step"]
            c4.append(brief(r, keys=("B", "us_per_layer", "us_per_step", "GBps", "frac_of_copy_peak",
                                     "distinct_experts", "layers", "us_per_step_with_router")))
            log(f"48-layer step B={b}: {r['us_per_step']:.1f} us/step, {r['us_per_layer']:.2f} us/layer, "
                f"{r['GBps']:.0f} GB/s ({r['frac_of_copy_peak']:.1%}); with the router step "
                f"{rr['us_per_step']:.1f} us/step")
        extra["decode_step_48_layers"] = c4
        del deep
        torch.cuda.empty_cache()

        # wider expert shape: H=4096, I=1536, 8 layers
        S2d = mi.SHAPES["S2"]
        t0 = time.time()
        L2 = mi.make_layer(mi.layer_seed("wide_layers", 0), S2d["H"], S2d["I"], S2d["E"])
        wide = [[up(a) for a in (L2.w_gate, L2.s_gate, L2.w_up, L2.s_up, L2.w_down, L2.s_down)]]
        del L2
        wide += [distinct(wide[0], n) for n in range(1, 8)]
        torch.cuda.synchronize()
        log(f"wide layer ready in {time.time() - t0:.1f}s")
        c5 = []
        S2 = (S2d["H"], S2d["I"], S2d["E"], S2d["k"])
        for b in (1, 16, 32, 64):
            r = run_steps(wide, S2, b, args.sweep_steps // 2, 5, 32, seed=mi.routing_seed("wide_layers", b))
            r["frac_of_copy_peak"] = r["GBps"] / copy_gbps
            c5.append(brief(r))
            log(f"H=4096/I=1536 B={b}: {r['us_per_layer']:.2f} us/layer, {r['GBps']:.0f} GB/s "
                f"({r['frac_of_copy_peak']:.1%}); gate_up {r['gate_up_us']:.2f} us, down {r['down_us']:.2f} us "
                f"({r['kernels']})")
        extra["wide_shape_h4096_i1536"] = c5
        del wide
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        def oracle_passes(seconds, max_n, start):
            spent, byt, n = 0.0, 0, 0
            while n < max_n and (n == 0 or spent < seconds):
                seed = mi.routing_seed("batch_sweep", B)
                x = mi.make_x(seed, B, H, it=start + n)
                ids, w = mi.route_uniform(seed, B, E, k, it=start + n)
                c0 = time.perf_counter()
                oracle.layer(x, ids, w, *host_w)
                spent += time.perf_counter() - c0
                byt += layer_bytes(ids, H, I, k)["total"]
                n += 1
            return spent, byt, n

        cores = oracle.set_threads(0)
        spent, byt, n = oracle_passes(args.cpu_seconds, 64, 0)
        oracle.set_threads(1)   # one layer pass on one thread
        s1_spent, s1_byt, _ = oracle_passes(0.0, 1, n)
        oracle.set_threads(0)
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
        except OSError:
            pass
        cpu = {"value": round(byt / spent / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "cpu_model": model,
               "sample": f"{n} layer passes at B={B} (H=2048, E=128, k=8, I=768, uniform routing), "
                         f"FP64 C oracle on {cores} threads, {spent:.1f} s, {spent / n * 1e3:.1f} ms/layer",
               "single_thread": {"value": round(s1_byt / s1_spent / 1e9, 4), "unit": "GB/s",
                                 "ms_per_layer": round(s1_spent * 1e3, 1),
                                 "sample": f"1 layer pass at B={B} on 1 thread"}}
        log(f"cpu oracle ({model}): {cpu['value']} GB/s on {cores} threads ({spent / n * 1e3:.1f} ms/layer); "
            f"1 thread {s1_spent * 1e3:.0f} ms/layer")

    # roofline position of both kernels at the headline (HBM-bound: algorithmic bytes
    # per launch / event-timed launch duration, against the published 8 TB/s); the
    # dominant one (gate/up, 2/3 of the bytes) is `roofline`
    gu_variant = mg.moe_decode_gate_up_plan(B, H, I, E, k)[0]
    dn_variant = mg.moe_decode_down_plan(B, H, I, E, k)[0]
    names = {
        "gate_up": {mg.MOE_GATE_UP_PER_SLOT: "moe_gate_up_3d_batched_w64",
                    mg.MOE_GATE_UP_EXPERT_GROUPED: "moe_gate_up_expert_grouped_w64",
                    mg.MOE_GATE_UP_EXPERT_GROUPED_MFMA: "moe_gate_up_grouped_mfma_w64"}[gu_variant],
        "down": {mg.MOE_DOWN_PER_TOKEN: "moe_down_3d_batched_w64",
                 mg.MOE_DOWN_EXPERT_GROUPED: "moe_down_expert_grouped_w64",
                 mg.MOE_DOWN_EXPERT_GROUPED_MFMA: "moe_down_grouped_mfma_w64"}[dn_variant],
    }

    # the counters in profiles/traffic.json hold for this shape and routing only
    traffic_workload = {"B": B, "H": H, "I": I, "E": E, "k": k, "routing": "uniform"}

    def roofline(which):
        gbps = kern[f"{which}_GBps"]
        return {"bound": "hbm", "kernel": names[which], "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(which, names[which], traffic_workload),
                "algorithmic_bytes_per_launch": round(kern[f"{which}_bytes_per_launch"]),
                "us_per_launch": round(kern[f"{which}_us"], 3)}

    roof = roofline("gate_up")
    out = {
        "metric": METRIC,
        "value": round(main_res["GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["seconds"] / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"single MoE decode layer, B={B}, H=2048, E=128, top-8, I=768, MXFP8 E4M3/E8M0-per-32 "
                               f"weights, bf16 activations, uniform routing (fresh per step), "
                               f"{args.copies} weight copies cycled",
                   "B": B, "H": H, "E": E, "k": k, "I": I},
        "us_per_layer": round(main_res["us_per_layer"], 3),
        "us_per_layer_p10": round(main_res["us_per_layer_p10"], 3),
        "us_per_layer_p90": round(main_res["us_per_layer_p90"], 3),
        "timed_replays": main_res["replays"],
        "frac_of_copy_peak": round(main_res["GBps"] / copy_gbps, 4),
        "copy_peak_GBps": round(copy_gbps, 1),
        "read_peak_GBps": round(read_gbps, 1),
        "peak_by_size": peak_by_size,
        "distinct_experts_mean": round(main_res["distinct_experts"], 2),
        "kernels_us": {"gate_up": round(kern["gate_up_us"], 3), "down": round(kern["down_us"], 3)},
        "vector_units_only": {"us_per_layer": round(vec["us_per_layer"], 3), "GBps": round(vec["GBps"], 1),
                              "frac_of_copy_peak": round(vec["GBps"] / copy_gbps, 4),
                              "kernels": "moe_gate_up_expert_grouped_w64 + moe_down_expert_grouped_w64"},
        "roofline": roof,
        "roofline_down": roofline("down"),
        "cpu_baseline": cpu,
        "sweep": sweep,
        **extra,
        "wall_seconds_timed": round(main_res["wall_seconds"], 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
