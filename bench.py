"""Throughput of the fused MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]

A step is one ``moe_fused_forward`` over one batch of T tokens: router, sort
by expert, gate/up product with SiLU-and-mul, down product, weighted combine
(and both E4M3 quantisations when the experts are FP8).  Inputs are seeded,
synthetic and resident in HBM before the timed region.  The default workload
is the bfloat16 decode layer H=4096, I=14336, E=8, K=2 at T=64 tokens.

Printed: ONE JSON line with tokens/s, the whole-layer algorithmic HBM rate,
the roofline of the dominant kernel (timed with the library's stage events on
the stream the kernels run on), per-stage times, a parity check of the same
code on a sub-batch against the CPU oracle, and the oracle's own rate on that
sub-batch (``cpu_baseline``).
"""

import argparse
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0                          # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # dense MFMA
METRIC = "MoE-layer tokens/s + HBM GB/s % peak (decode T=1..64); fp8 TFLOP/s (T=4096)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="bf16_decode")
    ap.add_argument("--T", type=int, default=None,
                    help="tokens per batch (default: the largest decode batch, "
                         "or 4096 for the prefill workload)")
    ap.add_argument("--scales", choices=("tensor", "row"), default="tensor",
                    help="FP8 workloads: one scale per expert tensor (and per activation "
                         "tensor), or one per weight row and per activation row")
    ap.add_argument("--fp8-format", choices=("e4m3", "e5m2"), default="e4m3",
                    help="FP8 workloads: the code format of weights and activations")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work the cpu_baseline sample aims at")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: read two rocprofv3 --pmc result folders (FETCH_SIZE, "
                         "WRITE_SIZE) of this same command with --copy-calib-mib, and store "
                         "the dominant kernel's HBM bytes per call in profiles/traffic.json")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the secondary timing of the same steps replayed from a HIP graph")
    ap.add_argument("--no-first-call-check", action="store_true",
                    help="skip calling the layer at never-seen token counts (1..64, 100, 257, "
                         "4096, shuffled) after the measurement, each first call compared with "
                         "the p95 of the following ten (nothing is compiled at run time)")
    ap.add_argument("--no-copy-bw", action="store_true",
                    help="skip measuring the device copy rate (the second HBM denominator)")
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="default workload only: skip the FP8 decode (T=64), FP8 prefill "
                         "(T=4096) and inverse-RoPE entries")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="before the layer, copy this many MiB once with a plain "
                         "device copy (a known-size reference for HBM counters)")
    return ap.parse_args()


def source_digest():
    """sha256 of the HIP sources with comments and blank lines removed; traffic
    counters are valid for one digest (a comment edit keeps them)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "moe_layer_05_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
        h.update(f.encode() + b"\0" + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


def traffic_key(workload, T, scales, fmt="e4m3"):
    return (f"{workload}/T{T}" + ("/row_scales" if scales == "row" else "")
            + ("/e5m2" if fmt == "e5m2" else ""))


def load_traffic(workload, T, kernel, scales="tensor", fmt="e4m3"):
    """HBM bytes per launch of ``kernel`` from the committed counter runs, or
    None when there are none for this workload or the kernels have changed."""
    try:
        with open(TRAFFIC_FILE) as fh:
            db = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = db.get(traffic_key(workload, T, scales, fmt))
    if not rec or rec.get("source_digest") != source_digest() or rec.get("kernel") != kernel:
        return None
    return rec.get("bytes_per_launch")


STAGE_KERNELS = {"gate_up": re.compile(r"moe_gemm_\w+_kernel<0,"),
                 "down": re.compile(r"moe_gemm_\w+_kernel<1,|moe_down_small_kernel")}


def read_counter(folder, counter):
    """{dispatch id: (kernel name, summed value)} of one rocprofv3 --pmc run."""
    import csv
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {folder}, found {len(files)}")
    out = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def record_traffic(args):
    """HBM bytes per call of the dominant stage from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    calibration kernel that reads and writes a known number of bytes."""
    if not args.copy_calib_mib:
        raise SystemExit("--record-traffic needs the --copy-calib-mib of the profiled runs")
    from moe_layer_05_amd import workloads
    cfg = workloads.CONFIGS[args.workload]
    T = args.T or (4096 if args.workload == "fp8_prefill_zipf" else max(cfg.Ts))
    n = float(args.copy_calib_mib << 20)
    rec = {"kernel": "gate_up", "source_digest": source_digest()}
    for folder, counter, key in ((args.record_traffic[0], "FETCH_SIZE", "fetch"),
                                 (args.record_traffic[1], "WRITE_SIZE", "write")):
        disp = read_counter(folder, counter)
        calib = [v for name, v in disp.values() if "bitwise_not" in name]
        calls = sum(1 for name, _ in disp.values()
                    if "router_kernel" in name or "front_kernel" in name)
        stage = [v for name, v in disp.values() if STAGE_KERNELS["gate_up"].search(name)]
        if len(calib) != 1 or calls == 0 or not stage:
            raise SystemExit(f"{folder}: calibration {len(calib)}, calls {calls}, "
                             f"stage dispatches {len(stage)}")
        factor = calib[0] * 1024.0 / n           # counter bytes per real byte
        rec[f"{key}_factor"] = round(factor, 4)
        rec[f"{key}_bytes_per_call"] = round(sum(stage) * 1024.0 / factor / calls)
        rec["calls"] = calls
    rec["bytes_per_launch"] = rec["fetch_bytes_per_call"] + rec["write_bytes_per_call"]
    try:
        with open(TRAFFIC_FILE) as fh:
            db = json.load(fh)
    except (OSError, ValueError):
        db = {}
    key = traffic_key(cfg.name, T, args.scales, args.fp8_format)
    db[key] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({key: rec}))


class Work:
    """Sizes and algorithmic work of one call, from the actual routing."""

    def __init__(self, cfg, T, ids, rows=False):
        import numpy as np
        self.cfg, self.T = cfg, T
        fp8 = cfg.wdtype == "fp8"
        rows = rows and fp8
        bw = 1 if fp8 else 2
        H, I, E, K = cfg.H, cfg.I, cfg.E, cfg.K
        P = T * K
        self.active = int(np.unique(ids).size)
        w13_e, w2_e = 2 * I * H * bw, H * I * bw
        # weight scales per expert: one per tensor, or one per row (float32)
        sc13, sc2 = ((2 * I * 4, H * 4) if rows else (4, 4)) if fp8 else (0, 0)
        # activation scales read by each product: per token row of x, per pair row of a
        sx, sa = (T * 4, P * 4) if rows else (0, 0)
        # whole layer: active experts' weights (+ scales), x, logits, out
        self.layer_bytes = (self.active * (w13_e + w2_e + sc13 + sc2) + T * H * 2 + T * E * 4
                            + T * H * 2)
        self.layer_flops = 6.0 * H * I * P
        # gate/up kernel: its experts' w13, the x rows (E4M3 codes or bf16)
        # and the intermediate it writes (float32 for the FP8 path, bf16 else)
        self.stage_bytes = {
            "gate_up": self.active * (w13_e + sc13) + T * H * (1 if fp8 else 2) + sx
                       + P * I * (4 if fp8 else 2),
            "down": self.active * (w2_e + sc2) + P * I * (1 if fp8 else 2) + sa + P * H * 4
                    + P * 4,
        }
        self.stage_flops = {"gate_up": 4.0 * H * I * P, "down": 2.0 * H * I * P}
        self.kind = "fp8" if fp8 else "bf16"


def roofline(work, stage, us):
    """Roofline entry of one kernel: whichever of HBM and MFMA bounds it."""
    b = work.stage_bytes[stage]
    f = work.stage_flops[stage]
    peak_f = PEAK_TFLOPS[work.kind]
    t_hbm = b / (PEAK_HBM_GBPS * 1e9)
    t_mfma = f / (peak_f * 1e12)
    s = us * 1e-6
    if t_mfma > t_hbm:
        ach = f / s / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(ach / peak_f, 4)}
    ach = b / s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBPS, 4)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def host_weights(w):
    """Indexable per-expert host copies for the oracle (one expert at a time)."""
    import torch

    class Experts:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            x = self.t[int(e)].to("cpu")
            return x.numpy() if x.dtype == torch.uint8 else x.float().numpy()

    return Experts(w)


def oracle_and_parity(cfg, m, w, tk, budget, scales="tensor", fmt="e4m3"):
    """Time the CPU oracle (float32 products, BLAS on every host core) on
    sub-batches of the first n tokens (n doubling while the last run stays well
    inside ``budget`` seconds), and compare the library on the same sub-batch
    with that run's output (float32 and float64 oracle outputs differ by
    <= 1e-5 relative, a pinned bound).  Returns (cpu_baseline, parity)."""
    import numpy as np
    import torch
    from oracle import moe as omoe

    fp8 = cfg.wdtype == "fp8"
    T = tk["x"].shape[0]
    kw = dict(w13=host_weights(w["w13"]), w2=host_weights(w["w2"]),
              wdtype="fp8" if fp8 else "float")
    if fp8:
        kw["w13_scale"] = w["w13_scale"].cpu().numpy()
        kw["w2_scale"] = w["w2_scale"].cpu().numpy()
    n, last = 1, None
    while True:
        x = tk["x"][:n].contiguous()
        lg = tk["logits"][:n].contiguous()
        xh = x.float().cpu().numpy()
        lh = lg.cpu().numpy()
        t0 = time.perf_counter()
        ref, parts = omoe.moe_forward(xh, lh, K=cfg.K, return_parts=True, dtype=np.float32,
                                      act_scales=scales if fp8 else "tensor",
                                      fp8_format=fmt, **kw)
        dt = time.perf_counter() - t0
        last = (n, dt, ref, parts, x, lg)
        log(f"oracle sub-batch of {n} tokens: {dt:.2f} s")
        if n >= T or dt * 2.3 > budget:
            break
        n = min(T, 2 * n)
    n, dt, ref, parts, x, lg = last
    # a whole batch that runs in a few seconds is run again until the sample
    # holds about half the budget of oracle work; the rate is over all runs
    runs, total = 1, dt
    if n >= T:
        xh, lh = x.float().cpu().numpy(), lg.cpu().numpy()
        while total < budget / 2 and runs < 16:
            t0 = time.perf_counter()
            omoe.moe_forward(xh, lh, K=cfg.K, act_scales=scales if fp8 else "tensor",
                             fp8_format=fmt, dtype=np.float32, **kw)
            total += time.perf_counter() - t0
            runs += 1
        log(f"oracle: {runs} runs of the {n}-token batch, {total:.2f} s")
    out, ids, _ = m(x, lg, return_topk=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    err = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
    ids_ok = bool(np.array_equal(ids.cpu().numpy(), parts["ids"]))
    cpu = {"value": round(n * runs / total, 3), "unit": "tokens/s", "cores": blas_threads(),
           "kind": "oracle",
           "sample": f"first {n} of the {T} tokens run as their own batch through the "
                     f"numpy oracle with float32 products (same weights), {runs} run(s), "
                     f"{total:.2f} s"}
    parity = {"tokens": n, "ids_bit_exact": ids_ok, "max_rel_err": err, "tol": 1e-2,
              "ok": ids_ok and err <= 1e-2}
    return cpu, parity


def graph_replay(mods, x, lg, out, steps):
    """Secondary timing: one call per weight copy captured into a HIP graph
    (torch.cuda.CUDAGraph), the graphs replayed in turn for the same number of
    steps; every replay's output is checked against the eager call's."""
    import torch
    torch.cuda.synchronize()
    ref = [m(x, lg).clone() for m in mods]                 # eager results per copy
    outs = [torch.empty_like(out) for _ in mods]
    graphs = []
    for m, o in zip(mods, outs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            m(x, lg, out=o)
        graphs.append(g)
    torch.cuda.synchronize()
    ok = True
    for i, g in enumerate(graphs * 2):                      # replays with checks between
        g.replay()
        torch.cuda.synchronize()
        j = i % len(graphs)
        ok = ok and bool(torch.equal(outs[j], ref[j]))
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    return {"ms_per_step": round(ms, 4), "replays_match_eager": ok}


def first_call_check(cfg, m, T_done, dev, stream):
    """First call at each never-seen token count against the p95 of the ten
    calls that follow it (same process, workspace sized beforehand so no call
    allocates).  A 512 MiB buffer is overwritten before every call, so the
    first call and the later ones all start with the same cold caches (without
    it the later calls find the weights of the first in the last-level cache).
    The library compiles nothing at run time, so a first call costs what a
    later one does."""
    import random
    import numpy as np
    import torch
    from moe_layer_05_amd import workloads
    Ts = [t for t in list(range(1, 65)) + [100, 257, 4096] if t != T_done]
    random.Random(0).shuffle(Ts)
    m.workspace(max(Ts), dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ratios = []
    for t in Ts:
        tk = workloads.make_tokens(cfg, t, seed=1, device=dev)
        out = torch.empty(t, cfg.H, dtype=torch.bfloat16, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(11)]
        torch.cuda.synchronize()
        for a, b in evs:
            flush.zero_()
            a.record(stream)
            m(tk["x"], tk["logits"], out=out)
            b.record(stream)
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        ratios.append((us[0] / float(np.percentile(us[1:], 95)), t))
    del flush
    worst = max(ratios)
    r = np.array([q for q, _ in ratios])
    return {"t_values": len(Ts), "caches_flushed_before_each_call": True,
            "within_p95": int((r <= 1.0).sum()), "within_1.05x_p95": int((r <= 1.05).sum()),
            "median_first_over_p95": round(float(np.median(r)), 3),
            "max_first_over_p95": round(worst[0], 3), "at_T": worst[1]}


def cpu_info():
    """Host description for the CPU baseline: logical CPUs usable by this
    process, all logical CPUs, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": usable, "logical_cpus": os.cpu_count(), "cpu_model": model}


def copy_bandwidth(dev, mib=2048, reps=20):
    """Measured device copy rate (bytes read + written per second) of a plain
    torch copy of ``mib`` MiB: the secondary denominator of the HBM rooflines."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    import numpy as np
    ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def event_floor(stream):
    """What a pair of back-to-back event records reads with no kernel between
    them (the markers' own stream time)."""
    import numpy as np
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(50)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in pairs]))


def measure_layer(cfg, T, w, steps, warmup, dev, copy_gbps, rows=False, fmt="e4m3",
                  copies_max=8):
    """Time ``steps`` calls of the fused layer on one batch; returns the bench
    fields of one workload (rate, layer and dominant-kernel rooflines, stage
    breakdown) and the layer objects for later checks."""
    import numpy as np
    import torch
    import moe_layer_05_amd as mm
    from moe_layer_05_amd import binding, workloads

    tk = workloads.make_tokens(cfg, T, seed=0, device=dev)
    wbytes = w["w13"].numel() * w["w13"].element_size() + w["w2"].numel() * w["w2"].element_size()
    # Rotate weight copies when one set could stay in the 256 MB last-level
    # cache between steps, so every step streams its experts from HBM.
    copies = 1 if wbytes >= (1 << 30) else min(copies_max, math.ceil((2 << 30) / wbytes))
    sets = [w] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
                  for _ in range(copies - 1)]
    mods = [mm.FusedMoE(s["w13"], s["w2"], cfg.K, s.get("w13_scale"), s.get("w2_scale"),
                        fp8_format=fmt) for s in sets]
    x, lg = tk["x"], tk["logits"]
    out = torch.empty(T, cfg.H, dtype=torch.bfloat16, device=dev)
    _, ids, _ = mods[0](x, lg, out=out, return_topk=True)
    torch.cuda.synchronize()
    work = Work(cfg, T, ids.cpu().numpy(), rows)

    nst = len(binding.STAGES)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        mods[i % copies](x, lg, out=out)
    torch.cuda.synchronize()

    # Timed region: K steps; in every `every`-th of them the library records
    # two events around the gate/up kernel (the dominant one: two thirds of
    # the weight bytes and of the flops) on the stream that kernel runs on.
    # An event record costs the stream about 3 us here (measured: events
    # around gate/up in every step add 6-7 us per step at every decode
    # shape, in every 8th step about 1 us), so the markers sit in a sample
    # of the steps (at least 10 of them) rather than in all.
    G0, G1 = binding.STAGES.index("gate_up"), binding.STAGES.index("gate_up") + 1
    every = max(1, min(8, steps // 10))
    evs = []
    for i in range(steps):
        if i % every:
            evs.append(None)
            continue
        row = [None] * (nst + 1)
        row[G0] = torch.cuda.Event(enable_timing=True)
        row[G1] = torch.cuda.Event(enable_timing=True)
        row[G0].record(stream)                # creates the events before the timed region
        row[G1].record(stream)
        evs.append(row)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        mods[i % copies](x, lg, out=out, events=evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom = "gate_up"
    dom_raw_us = float(np.mean([e[G0].elapsed_time(e[G1]) * 1e3 for e in evs if e is not None]))
    # The kernel's duration is the event pair's reading as is.  What a pair
    # of back-to-back records reads with nothing between them is reported
    # beside it but not taken off: that floor varies between runs (4.4 us
    # typically, 8.1 in one run), and the raw readings agree with the kernel
    # traces within a few percent (bf16 T = 64 gate/up 321.0 vs 317.8 us,
    # TP8 slice T = 64 42.9 vs 42.0, fp8 T = 1 39.8 vs 37.0).
    floor_us = event_floor(stream)
    dom_us = dom_raw_us

    # After the timed region: a breakdown with every stage boundary recorded
    # (each record adds a few microseconds, so these steps are not the rate).
    nb = min(steps, 50)
    bevs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(nb)]
    for row in bevs:
        for ev in row:
            ev.record(stream)
    torch.cuda.synchronize()
    for i in range(nb):
        mods[i % copies](x, lg, out=out, events=bevs[i])
    torch.cuda.synchronize()
    stage_us = {}
    for s_, name in enumerate(binding.STAGES):
        d = [bevs[i][s_].elapsed_time(bevs[i][s_ + 1]) * 1e3 for i in range(nb)]
        stage_us[name] = round(float(np.mean(d)), 2)
    step_us = [bevs[i][0].elapsed_time(bevs[i][nst]) * 1e3 for i in range(nb)]

    ms = elapsed / steps * 1e3
    roof = roofline(work, dom, dom_us)
    roof["scope"] = "dominant kernel only (gate/up product); the layer's own rate is under layer"
    roof["kernel"] = dom
    roof["kernel_us"] = round(dom_us, 2)
    roof["event_pair_floor_us"] = round(floor_us, 2)
    roof["event_timed_steps"] = sum(1 for e in evs if e is not None)
    roof["traffic"] = load_traffic(cfg.name, T, dom, "row" if rows else "tensor", fmt)
    roof["algorithmic_bytes"] = work.stage_bytes[dom]
    roof["algorithmic_flops"] = work.stage_flops[dom]
    if roof["bound"] == "hbm" and copy_gbps:
        roof["copy_gbps"] = copy_gbps
        roof["frac_of_copy"] = round(roof["achieved"] / copy_gbps, 4)
    gbps = work.layer_bytes / (ms * 1e-3) / 1e9
    layer = {"algorithmic_bytes": work.layer_bytes, "hbm_gbps": round(gbps, 1),
             "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
             "tflops": round(work.layer_flops / (ms * 1e-3) / 1e12, 2),
             "mfma_frac": round(work.layer_flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS[work.kind], 4),
             "step_us_with_all_stage_events_p50": round(float(np.percentile(step_us, 50)), 2),
             "step_us_with_all_stage_events_p95": round(float(np.percentile(step_us, 95)), 2)}
    if copy_gbps:
        layer["frac_of_copy"] = round(gbps / copy_gbps, 4)
    fields = {
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "dtype": f"fp8_{fmt}" if cfg.wdtype == "fp8" else "bf16",
        "config": {"workload": cfg.name, "T": T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "K": cfg.K, "weights": "fp8" if cfg.wdtype == "fp8" else "bf16",
                   "routing": cfg.routing,
                   "fp8_scales": ("row" if rows else "tensor") if cfg.wdtype == "fp8" else None,
                   "fp8_format": fmt if cfg.wdtype == "fp8" else None,
                   "active_experts": work.active, "weight_copies": copies},
        "roofline": roof,
        "layer": layer,
        "stages_us": stage_us,
    }
    return fields, mods, tk, out


def sub_batch_parity(cfg, m, w, tk, n, scales="tensor", fmt="e4m3"):
    """The library against the oracle on the first n tokens run as their own
    batch (ids bit-exact, output within 1e-2)."""
    import numpy as np
    import torch
    from oracle import moe as omoe
    fp8 = cfg.wdtype == "fp8"
    kw = dict(w13=host_weights(w["w13"]), w2=host_weights(w["w2"]),
              wdtype="fp8" if fp8 else "float")
    if fp8:
        kw["w13_scale"] = w["w13_scale"].cpu().numpy()
        kw["w2_scale"] = w["w2_scale"].cpu().numpy()
    x, lg = tk["x"][:n].contiguous(), tk["logits"][:n].contiguous()
    ref, parts = omoe.moe_forward(x.float().cpu().numpy(), lg.cpu().numpy(), K=cfg.K,
                                  return_parts=True, act_scales=scales if fp8 else "tensor",
                                  fp8_format=fmt, workers=8, **kw)
    out, ids, _ = m(x, lg, return_topk=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    err = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))
    ids_ok = bool(np.array_equal(ids.cpu().numpy(), parts["ids"]))
    return {"tokens": n, "ids_bit_exact": ids_ok, "max_rel_err": err, "tol": 1e-2,
            "ok": ids_ok and err <= 1e-2}


def one_thread_oracle(cfg, w, tk, scales="tensor", fmt="e4m3"):
    """Seconds of the oracle (float32 products) on token 0 alone with one BLAS
    thread."""
    from threadpoolctl import threadpool_limits
    from oracle import moe as omoe
    import numpy as np
    fp8 = cfg.wdtype == "fp8"
    kw = dict(w13=host_weights(w["w13"]), w2=host_weights(w["w2"]),
              wdtype="fp8" if fp8 else "float")
    if fp8:
        kw["w13_scale"] = w["w13_scale"].cpu().numpy()
        kw["w2_scale"] = w["w2_scale"].cpu().numpy()
    x = tk["x"][:1].float().cpu().numpy()
    lg = tk["logits"][:1].cpu().numpy()
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        omoe.moe_forward(x, lg, K=cfg.K, dtype=np.float32, act_scales=scales, fp8_format=fmt,
                         **kw)
        return round(time.perf_counter() - t0, 3)


def measure_inv_rope(dev, copy_gbps, T=4096, steps=100):
    """The attention-side kernel (inverse rotary embedding + per-head FP8):
    bytes it must move per launch over its event-timed duration, and parity
    of the same call against the oracle."""
    import numpy as np
    import torch
    import moe_layer_05_amd as mm
    from moe_layer_05_amd import workloads
    from oracle import rope as orope
    cfg = workloads.ROPE_CONFIGS["inv_rope_tp8"]
    d = workloads.make_heads(cfg, T, seed=0, device=dev)
    table = workloads.rope_table(cfg.max_pos, cfg.R)
    tab = table.to(dev)
    x, pos = d["x"], d["positions"]
    codes = torch.empty(T, cfg.NH, cfg.D, dtype=torch.uint8, device=dev)
    scales = torch.empty(T, cfg.NH, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # rotate over copies of x so the timed launches read HBM, not the caches
    xs = [x] + [x.clone() for _ in range(7)]
    for i in range(10):
        mm.inv_rope_fp8_quant_per_head(xs[i % 8], pos, tab, cfg.R, codes=codes, scales=scales)
    # one event pair around `steps` back-to-back launches: a ~10 us kernel is
    # short beside an event pair's own few microseconds, which this spreads
    # over all the launches (back-to-back launches abut in kernel traces)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        mm.inv_rope_fp8_quant_per_head(xs[i % 8], pos, tab, cfg.R, codes=codes, scales=scales)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    rows = T * cfg.NH
    # x read, codes and scales written, positions read, one table row per token
    nbytes = rows * cfg.D * 2 + rows * cfg.D + rows * 4 + T * 8 + T * cfg.R * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    mm.inv_rope_fp8_quant_per_head(x, pos, tab, cfg.R, codes=codes, scales=scales)
    torch.cuda.synchronize()
    rc, rs = orope.inv_rope_fp8_quant_per_head(x.float().cpu().numpy(), pos.cpu().numpy(),
                                               table.numpy(), cfg.R, cfg.interleaved)
    exact = bool(np.array_equal(codes.cpu().numpy(), rc)
                 and np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32)))
    roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None, "kernel_us": round(us, 2),
            "algorithmic_bytes": nbytes}
    if copy_gbps:
        roof["copy_gbps"] = copy_gbps
        roof["frac_of_copy"] = round(gbps / copy_gbps, 4)
    return {"metric": "inverse RoPE + per-head FP8 quantisation, heads/s", "T": T,
            "value": round(rows / (us * 1e-6), 1), "unit": "heads/s",
            "config": {"workload": cfg.name, "NH": cfg.NH, "D": cfg.D, "R": cfg.R,
                       "interleaved": cfg.interleaved},
            "roofline": roof, "parity": {"codes_and_scales_bit_exact": exact}}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.record_traffic:
        record_traffic(args)
        return
    import torch

    import moe_layer_05_amd as mm
    from moe_layer_05_amd import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mm.lib()                                  # fail loudly if the library is missing

    cfg = workloads.CONFIGS[args.workload]
    T = args.T or (4096 if args.workload == "fp8_prefill_zipf" else max(cfg.Ts))
    log(f"workload {cfg.name} T={T} H={cfg.H} I={cfg.I} E={cfg.E} K={cfg.K} {cfg.wdtype}")

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)       # one elementwise kernel: n bytes in, n out
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: {args.copy_calib_mib} MiB read + written once")

    copy_gbps = None if args.no_copy_bw else copy_bandwidth(dev)
    log(f"device copy rate {copy_gbps} GB/s")
    wdtype = "bf16" if cfg.wdtype == "float32" else cfg.wdtype
    rows = args.scales == "row" and wdtype == "fp8"
    fmt = args.fp8_format
    w = workloads.make_weights(cfg, seed=0, device=dev, wdtype=wdtype,
                               scales="row" if rows else "tensor", fp8_format=fmt)
    fields, mods, tk, out = measure_layer(cfg, T, w, args.steps, args.warmup, dev, copy_gbps,
                                          rows, fmt)

    graph = None if args.no_graph else graph_replay(mods, tk["x"], tk["logits"], out, args.steps)
    first_call = None
    if not args.no_first_call_check:
        first_call = first_call_check(cfg, mods[0], T, dev, torch.cuda.current_stream())

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = oracle_and_parity(cfg, mods[0], w, tk, args.cpu_budget,
                                        "row" if rows else "tensor", fmt)
        cpu.update(cpu_info())
        cpu["threads"] = cpu["cores"]
        if T > 1 and cfg.name in ("bf16_decode", "fp8_decode"):
            cpu["one_thread_T1_s"] = one_thread_oracle(cfg, w, tk, "row" if rows else "tensor",
                                                       fmt)
    del mods

    secondary = []
    if args.secondary and args.workload == "bf16_decode" and not rows and fmt == "e4m3":
        # the metric's FP8 half: decode at 64 tokens and the skewed prefill,
        # on one set of E4M3 weights (the two workloads share the expert shapes)
        del w
        torch.cuda.empty_cache()
        c8 = workloads.CONFIGS["fp8_decode"]
        w8 = workloads.make_weights(c8, seed=0, device=dev, wdtype="fp8")
        f8, m8, tk8, _ = measure_layer(c8, 64, w8, args.steps, args.warmup, dev, copy_gbps)
        f8["parity"] = sub_batch_parity(c8, m8[0], w8, tk8, 2)
        f8["cpu_baseline_one_thread_T1_s"] = one_thread_oracle(c8, w8, tk8)
        secondary.append(f8)
        del m8
        cp = workloads.CONFIGS["fp8_prefill_zipf"]
        fp, mp, _, _ = measure_layer(cp, 4096, w8, max(10, args.steps // 4),
                                     max(3, args.warmup // 4), dev, copy_gbps)
        fp["parity"] = {"covered_by": "tests/test_gpu_parity.py::"
                                      "test_fused_fp8_prefill_zipf_sampled (24 sampled tokens "
                                      "of this batch and every intermediate of the call)"}
        secondary.append(fp)
        del mp, w8
        torch.cuda.empty_cache()
        secondary.append(measure_inv_rope(dev, copy_gbps))

    line = {
        "metric": METRIC,
        "value": fields["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fields["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fields["dtype"],
        "data": "synthetic",
        "config": fields["config"],
        "roofline": fields["roofline"],
        "cpu_baseline": cpu,
        "layer": fields["layer"],
        "stages_us": fields["stages_us"],
        "parity": parity,
        "graph": graph,
        "first_call": first_call,
        "copy_gbps": copy_gbps,
        "secondary": secondary,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
