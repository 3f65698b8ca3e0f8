"""Benchmark: block-sparse decode attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long-128k]

One step = one pass of the decode hot path for one attention layer over one
batch: block representatives of blocks that filled (none at the measured
workload's steps), then scoring, selection and the sparse decode, either as
the one fused launch nsa_decode_step (default) or as nsa_select_blocks +
nsa_sparse_decode (--path split).  Inputs are seeded synthetic tensors already
resident in HBM when timing starts.  Steps rotate over R independent layer
instances (own pools, representatives, state and workspaces; R x working set
>= 1 GiB) so that the ~256 MB Infinity Cache cannot hold the step's bytes and
the figures are HBM figures.

Prints one JSON line (rank 0, N = 1 only):
  value          decode tokens/s (batch / step time)
  roofline       the dominant kernel's algorithmic bytes per launch / its mean
                 launch duration from HIP events around each launch on its
                 stream (a second pass over the same steps, after the timed
                 one), against the 8 TB/s HBM peak; traffic = measured HBM
                 bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE
                 (scaled by a copy kernel of known size) when a record for the
                 current kernel source exists under profiles/, else null
  cpu_baseline   the CPU oracle (float64 NumPy) timed on a bounded sample of
                 the same workload's rows and steps, scaled to tokens/s
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
WORKLOADS = {"tiny-fp32": 0, "nosa-1b": 1, "sparda-8b": 2, "long-128k": 3, "early-stop": 4}
PREFILL_WORKLOADS = ("s2o-prefill-32k",)
KERNEL_SOURCES = {
    "select": "block_sparse_kv_nsa_amd/csrc/nsa_select.hip",
    "decode": "block_sparse_kv_nsa_amd/csrc/nsa_decode.hip",
    "step": "block_sparse_kv_nsa_amd/csrc/nsa_step.hip",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="long-128k",
                    choices=sorted(WORKLOADS) + list(PREFILL_WORKLOADS))
    ap.add_argument("--instances", type=int, default=0, help="layer instances to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle leg")
    ap.add_argument("--cpu-rows", type=int, default=8, help="rows sampled by the oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one float32 scale-by-one of MIB MiB (reads and writes MIB MiB) "
                         "before timing, the reference kernel for HBM byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter files of a "
                         "--copy-calibration run into profiles/<kernel>_<workload>_traffic.json")
    ap.add_argument("--calibration-mib", type=int, default=256,
                    help="the MIB of the --copy-calibration run read by --traffic-from")
    ap.add_argument("--path", default="fused", choices=("fused", "split"),
                    help="fused: one nsa_decode_step launch; split: nsa_select_blocks + "
                         "nsa_sparse_decode (the only path of the ordered early-stop mode)")
    ap.add_argument("--dense", action="store_true",
                    help="early-stop workload only: the dense reference, nsa_sparse_decode over "
                         "every full block with no scoring")
    ap.add_argument("--lookahead", action="store_true",
                    help="forecast workloads, two-call path: the layer instances form a stack; "
                         "layer l+1's selection runs on a second stream while layer l decodes "
                         "(it waits for layer l-1's decode, whose output the forecast of layer "
                         "l+1 is made from); value is this schedule's rate, the one-stream rate "
                         "is reported beside it")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps as one captured HIP graph instead of launching "
                         "them one by one (measured slower at short runs on this stack)")
    return ap.parse_args()


def code_only(text: str) -> str:
    """C++ source without its comments and blank lines: what the compiler
    sees, so that a comment edit does not count as a kernel change."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln.strip())


def source_hash(rel: str) -> str:
    h = hashlib.sha256()
    for part in (rel, "block_sparse_kv_nsa_amd/csrc/nsa_device.hpp",
                 "block_sparse_kv_nsa_amd/csrc/nsa_internal.hpp",
                 "block_sparse_kv_nsa_amd/csrc/nsa_attend.hpp"):
        with open(os.path.join(ROOT, part), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# algorithmic bytes: what the method must move per launch
# ----------------------------------------------------------------------------
def select_bytes(cfg, L: int) -> int:
    e = 2 if cfg.dtype == "bf16" else 4
    nb = L // 64
    reps = cfg.rows * nb * 4 * cfg.head_dim * e
    qv = (cfg.batch * cfg.num_kv_heads if cfg.mode.startswith("forecast") else cfg.batch * cfg.num_q_heads)
    qbytes = qv * cfg.head_dim * e
    out = cfg.rows * (cfg.k + 1) * 4
    state = cfg.rows * (2 * cfg.k_e + 1) * 4 if cfg.k_e else 0
    return reps + qbytes + out + state


def decode_bytes(cfg, L: int, n_blocks: int) -> int:
    e = 2 if cfg.dtype == "bf16" else 4
    tail = L % 64
    kv = cfg.rows * (n_blocks * 64 + tail) * cfg.head_dim * e * 2
    qo = 2 * cfg.batch * cfg.num_q_heads * cfg.head_dim * e
    idx = cfg.rows * (n_blocks + 1) * 4 * 2
    return kv + qo + idx


def traffic_from_profiles(workload: str, kernel: str):
    """Measured HBM bytes per launch from a committed rocprofv3 summary, if
    its kernel-source hash matches the current source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# GPU leg
# ----------------------------------------------------------------------------
def gpu_leg(args, cfg):
    import numpy as np
    import torch

    import workloads as W
    from block_sparse_kv_nsa_amd import SparseDecodeLayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    batch = W.build_batch(cfg)
    print(f"[bench] {cfg.name}: inputs drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    dense = args.dense
    fused = args.path == "fused" and not cfg.ordered and not dense
    L0 = cfg.seq_len(0)
    kp, vp = to_dev(batch.k_pool), to_dev(batch.v_pool)
    table = torch.from_numpy(batch.table).to(dev)
    logits = torch.from_numpy(batch.logits).to(dev)
    del batch
    pool_bytes = 2 * kp.numel() * kp.element_size()
    work = (decode_bytes(cfg, L0, cfg.nb0) if dense
            else select_bytes(cfg, L0) + decode_bytes(cfg, L0, cfg.k))
    R = args.instances or max(2, min(16, math.ceil((1 << 30) / max(1, work))))
    free = torch.cuda.mem_get_info()[0]
    R = max(1, min(R, int(0.6 * free // max(1, pool_bytes))))
    layers = []
    for r in range(R):
        lay = SparseDecodeLayer(batch=cfg.batch, num_q_heads=cfg.num_q_heads,
                                num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                                max_blocks_per_seq=cfg.max_blocks,
                                num_phys_blocks=cfg.num_phys_blocks, dtype=cfg.dtype,
                                mode=cfg.mode, k=cfg.k, k_e=cfg.k_e, ordered=cfg.ordered,
                                tau=cfg.tau, device=dev)
        lay.k_pool.copy_(kp)
        lay.v_pool.copy_(vp)
        lay.block_table.copy_(table)
        lay.evict_logits.copy_(logits)
        if not dense:
            first = torch.zeros(cfg.batch, dtype=torch.int32, device=dev)
            num = torch.full((cfg.batch,), cfg.nb0, dtype=torch.int32, device=dev)
            lay.update_reps(first, num, cfg.nb0)
        layers.append(lay)
    del kp, vp
    torch.cuda.synchronize()
    print(f"[bench] {R} layer instances ready ({pool_bytes / 2**30:.2f} GiB of K+V each)",
          file=sys.stderr, flush=True)

    # per-step inputs, device resident before timing
    steps = cfg.steps
    lens = [torch.full((cfg.batch,), cfg.seq_len(t), dtype=torch.int32, device=dev) for t in range(steps)]
    qs = [to_dev(W.queries(cfg, t)) for t in range(steps)]
    sel_q = ([to_dev(W.forecasts(cfg))] * steps) if cfg.mode.startswith("forecast") else qs
    fills = [(cfg.seq_len(t) % 64) == 0 for t in range(steps)]
    fill_first = [torch.full((cfg.batch,), cfg.seq_len(t) // 64 - 1, dtype=torch.int32, device=dev)
                  for t in range(steps)]
    ones = torch.ones(cfg.batch, dtype=torch.int32, device=dev)
    if dense:
        nbd = L0 // 64
        sel_all = torch.arange(nbd, dtype=torch.int32, device=dev).repeat(
            cfg.batch, cfg.num_kv_heads, 1).contiguous()
        nsel_all = torch.full((cfg.batch, cfg.num_kv_heads), nbd, dtype=torch.int32, device=dev)

    # every launch goes to the current stream (the capture stream while a
    # graph is being captured)
    def step(i, ev=None):
        lay = layers[i % R]
        t = i % steps
        lay.seq_lens = lens[t]
        if fills[t] and not dense:
            lay.update_reps(fill_first[t], ones, 1)
        if ev is not None:
            ev[0].record()
        if dense:
            lay.decode(qs[t], selected=sel_all, num_selected=nsel_all, max_selected=nbd,
                       early_stop=False)
            if ev is not None:
                ev[1].record()
                ev[2].record()
            return
        if fused:
            lay.step(sel_q[t], qs[t], cfg.seq_len(t))
            if ev is not None:
                ev[1].record()
                ev[2].record()
            return
        lay.select(sel_q[t], cfg.seq_len(t))
        if ev is not None:
            ev[1].record()
        lay.decode(qs[t])
        if ev is not None:
            ev[2].record()

    def check_status():
        if fused:
            for lay in layers:
                lay.check_step()     # raises when a wait of a fused step expired

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
    # set-up, untimed: one step per instance, so that each instance's first
    # call (the eviction-set update over the prefilled blocks) is never
    # timed, then steps for at least 0.25 s of device time so that the
    # device's clocks have left their idle state (they ramp up under load)
    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    t_set = time.perf_counter()
    i = 0
    while time.perf_counter() - t_set < 0.25:
        for _ in range(64):
            step(i)
            i += 1
        torch.cuda.synchronize()
    check_status()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    base = args.warmup
    graph = None
    if args.graph:
        # the K timed steps captured once as a HIP graph; one untimed replay
        # uploads it, the timed replay runs the same K steps again
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(base + i)
        graph.replay()
        torch.cuda.synchronize()
    lookahead = None
    if args.lookahead:
        lookahead = lookahead_pass(args, layers, sel_q, qs, lens, cfg, base)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # the device spins for a moment before the start event, so that the host
    # has submitted the timed work by the time the event is reached (the
    # submission latency is not part of the steps)
    torch.cuda._sleep(1_000_000)
    t_wall = time.perf_counter()
    start.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(base + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    check_status()
    del graph
    # per-kernel durations: the same steps again, launched one by one with
    # events around each launch on the launch stream (an event between
    # launches adds a small gap, so this pass is kept apart from the timed one)
    n_ev = min(args.steps, 1000)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for i in range(n_ev):
        step(base + args.steps + i, evs[i])
    torch.cuda.synchronize()
    check_status()
    sel_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ev
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / n_ev

    metrics = {}
    L_mid = cfg.seq_len(steps // 2)
    if dense:
        n_blocks = nbd
        sb, db = 0, decode_bytes(cfg, L_mid, n_blocks)
        metrics["blocks_attended"] = n_blocks
    elif cfg.ordered:
        n_star = torch.cat([lay.num_processed.flatten() for lay in layers]).float()
        n_blocks = n_star.mean().item()
        sb, db = select_bytes(cfg, L_mid), decode_bytes(cfg, L_mid, n_blocks)
        metrics["n_star"] = {"mean": round(n_blocks, 2), "min": int(n_star.min().item()),
                             "max": int(n_star.max().item()), "cap": cfg.k}
    else:
        n_blocks = layers[0].num_selected.float().mean().item()
        sb, db = select_bytes(cfg, L_mid), decode_bytes(cfg, L_mid, n_blocks)
        metrics.update(locality_metrics(layers[0], cfg, lens, sel_q, qs, fused))
    return dict(R=R, total_ms=total_ms, wall_s=wall, sel_ms=sel_ms, dec_ms=dec_ms,
                sel_bytes=sb, dec_bytes=db, n_blocks=n_blocks, fused=fused, dense=dense,
                graph=args.graph, metrics=metrics, lookahead=lookahead)


def lookahead_pass(args, layers, sel_q, qs, lens, cfg, base):
    """The layer instances as a stack of R layers, one token through it per
    R steps.  SparDA's forecast of layer l selects layer l+1's blocks (SparDA
    summary, "Trainierbare Lookahead Sparse-Selektion"), so layer l+1's
    selection can run while layer l decodes: it needs only the forecast,
    which is made from layer l's input, the output of layer l-1's decode.
    Step i (layer i mod R) therefore waits for its own selection; the
    selection of step i+1 runs on a second stream after step i-1's decode.
    Returns the timed rate of this schedule (K steps)."""
    import torch
    R = len(layers)
    steps = cfg.steps
    sel_stream = torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    ring = 4
    sel_done = [torch.cuda.Event() for _ in range(ring)]
    dec_done = [torch.cuda.Event() for _ in range(ring)]

    def select(i):
        lay, t = layers[i % R], i % steps
        lay.seq_lens = lens[t]
        lay.select(sel_q[t], cfg.seq_len(t), stream=sel_stream.cuda_stream)
        sel_done[i % ring].record(sel_stream)

    def run(first, n):
        select(first)
        for i in range(first, first + n):
            if i + 1 < first + n:
                if i > first:
                    sel_stream.wait_event(dec_done[(i - 1) % ring])
                select(i + 1)
            main.wait_event(sel_done[i % ring])
            layers[i % R].decode(qs[i % steps], stream=main.cuda_stream)
            dec_done[i % ring].record(main)

    run(base, 2 * R)  # untimed
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1_000_000)
    start.record(main)
    run(base, args.steps)
    end.record(main)
    torch.cuda.synchronize()
    return {"ms_per_step": start.elapsed_time(end) / args.steps,
            "schedule": "selection of layer l+1 on a second stream during layer l's decode"}


def locality_metrics(lay, cfg, lens, sel_q, qs, fused):
    """Untimed: one instance through every decode step of the workload again;
    after each step the library's residency diff gives the blocks to fetch
    (selected now, not resident after the previous step) and to release."""
    import torch
    import block_sparse_kv_nsa_amd as N
    if not hasattr(N, "nsa_residency_diff"):
        return {}
    dev = lay.device
    prev_sel = lay.selected.clone()
    prev_num = lay.num_selected.clone()
    prev_lens = lens[-1].clone()
    fetch = torch.empty_like(lay.selected)
    release = torch.empty((cfg.batch, cfg.num_kv_heads, cfg.k + 1), dtype=torch.int32, device=dev)
    n_fetch = torch.empty_like(lay.num_selected)
    n_release = torch.empty_like(lay.num_selected)
    gamma = torch.empty((cfg.batch, cfg.num_kv_heads), dtype=torch.float32, device=dev)
    g_min, f_tot, r_tot, f_max = 1.0, 0, 0, 0
    for t in range(cfg.steps):
        lay.seq_lens = lens[t]
        if fused:
            lay.step(sel_q[t], qs[t], cfg.seq_len(t))
        else:
            lay.select(sel_q[t], cfg.seq_len(t))
            lay.decode(qs[t])
        lay.residency_diff(prev_sel, prev_num, prev_lens, fetch, n_fetch, release, n_release, gamma)
        g_min = min(g_min, gamma.min().item())
        f_tot += int(n_fetch.sum().item())
        f_max = max(f_max, int(n_fetch.max().item()))
        r_tot += int(n_release.sum().item())
        prev_sel.copy_(lay.selected)
        prev_num.copy_(lay.num_selected)
        prev_lens = lens[t]
    if fused:
        lay.check_step()
    n = cfg.steps * cfg.rows
    return {"gamma_min": round(g_min, 4), "fetch_blocks_per_row_step": round(f_tot / n, 3),
            "fetch_blocks_max": f_max, "release_blocks_per_row_step": round(r_tot / n, 3),
            "gamma_bound": round(cfg.k_e / cfg.k, 4) if cfg.k_e else None}


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ----------------------------------------------------------------------------
def cpu_leg(args, cfg):
    import numpy as np

    import workloads as W
    from oracle import nsa_oracle as O

    host_cpus = os.cpu_count() or 1
    threads = min(host_cpus, 16)
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        limiter = None
    rows = [(b, g) for b in range(cfg.batch) for g in range(cfg.num_kv_heads)]
    rng = np.random.default_rng(5)
    order = [rows[i] for i in rng.permutation(len(rows))][:args.cpu_rows]
    # inputs and prefill of the sampled rows, outside the timed steps
    sample = []
    for (b, g) in order:
        ri = W.row_inputs(cfg, b, g)
        row = O.OracleRow(W.stored_to_f64(ri.keys, cfg.dtype), W.stored_to_f64(ri.values, cfg.dtype),
                          ri.logits.astype(np.float64), cfg.dtype, 1.0 / math.sqrt(cfg.head_dim),
                          mode=cfg.mode, k=cfg.k, k_e=cfg.k_e, ordered=cfg.ordered, tau=cfg.tau)
        if not args.dense:
            row.reps(cfg.nb0)
            if cfg.k_e:
                row.eviction_scores(cfg.nb0)
        qs = [W.stored_to_f64(W.query_row(cfg, b, g, t), cfg.dtype) for t in range(cfg.steps)]
        f = W.stored_to_f64(W.forecast_row(cfg, b, g), cfg.dtype) if cfg.mode.startswith("forecast") else None
        sample.append((row, qs, f))

    def one_pass():
        t0 = time.perf_counter()
        for row, qs, f in sample:
            for t in range(cfg.steps):
                L = cfg.seq_len(t)
                if args.dense:
                    O.dense_attention(qs[t], row.keys, row.values, L, row.scale)
                else:
                    row.step(L, qs[t], f=f)
        return time.perf_counter() - t0

    one_pass()                                   # warm-up
    # three timed bundles of repeated passes (a repeated step does the same
    # work: no block fills), each about a third of the budget
    probe = one_pass()
    per_bundle = max(1, int(args.cpu_seconds / 3 / max(probe, 1e-6)))
    times = []
    for _ in range(3):
        times.append(sum(one_pass() for _ in range(per_bundle)) / per_bundle)
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    per_pass = sorted(times)[1]
    per_row_step = per_pass / (len(sample) * cfg.steps)
    step_s = per_row_step * cfg.rows
    what = "dense attention over every cached token" if args.dense else "step"
    return {"value": cfg.batch / step_s, "unit": "tokens/s", "cores": threads,
            "host_cpus": host_cpus, "kind": "oracle",
            "sample": f"median of 3 timed bundles (after one warm-up pass) of {per_bundle} passes "
                      f"over the {cfg.steps} decode steps of {len(sample)} of {cfg.rows} rows "
                      f"({what}; float64 NumPy, one row at a time, BLAS limited to {threads} "
                      f"threads); scaled to all rows"}


# the kernels of one call (their per-launch counters are summed)
KERNEL_SYMBOLS = {"step": ("gang_kernel",), "select": ("score_kernel", "select_kernel"),
                  "decode": ("decode_kernel",)}
CALIBRATION_SYMBOL = "MulFunctor"


def counter_per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} of one counter from a rocprofv3
    counter-collection CSV (values summed over the rows of a dispatch)."""
    import csv
    per = {}
    with open(path, newline="") as fh:
        for rec in csv.DictReader(fh):
            if rec.get("Counter_Name") != counter:
                continue
            key = (rec["Kernel_Name"], rec.get("Dispatch_Id") or rec.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(rec["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def traffic_mode(args) -> int:
    fetch = counter_per_dispatch(args.traffic_from[0], "FETCH_SIZE")
    write = counter_per_dispatch(args.traffic_from[1], "WRITE_SIZE")
    known = args.calibration_mib * (1 << 20)

    def pick(table, sym):
        vals = [v for name, vs in table.items() if sym in name for v in vs]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named *{sym}* in the counter file")
        return sum(vals) / len(vals)

    f_cal, w_cal = pick(fetch, CALIBRATION_SYMBOL) * 1024, pick(write, CALIBRATION_SYMBOL) * 1024
    import workloads as W
    cfg = W.config(WORKLOADS[args.workload])
    workload = cfg.name + ("-dense" if args.dense else "")
    if args.dense:
        kernels = ["decode"]
    elif args.path == "fused" and not cfg.ordered:
        kernels = ["step"]
    else:
        kernels = ["select", "decode"]
    for kern in kernels:
        syms = KERNEL_SYMBOLS[kern]
        if kern == "decode" and cfg.ordered and not args.dense:
            syms = ("es_walk_kernel",)
        f_k = sum(pick(fetch, sym) for sym in syms) * 1024
        w_k = sum(pick(write, sym) for sym in syms) * 1024
        sym = "+".join(syms)
        rec = {
            "kernel": kern, "symbol": sym, "workload": workload,
            "fetch_bytes_raw": f_k, "write_bytes_raw": w_k,
            "calibration": {"kernel": CALIBRATION_SYMBOL, "bytes_each_way": known,
                            "fetch_bytes_raw": f_cal, "write_bytes_raw": w_cal,
                            "fetch_scale": known / f_cal, "write_scale": known / w_cal},
            "bytes_per_launch": f_k * known / f_cal + w_k * known / w_cal,
            "source_hash": source_hash(KERNEL_SOURCES[kern]),
            "files": list(args.traffic_from),
        }
        path = os.path.join(ROOT, "profiles", f"{kern}_{workload}_traffic.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
    return 0


def main():
    args = parse()
    if args.traffic_from:
        return traffic_mode(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this path shards by rows with no exchange, see the design notes)", file=sys.stderr)
        return 2
    if args.workload in PREFILL_WORKLOADS:
        return prefill_main(args)
    import workloads as W
    cfg = W.config(WORKLOADS[args.workload])
    if args.dense and not cfg.ordered:
        print("--dense is the early-stop workload's dense reference", file=sys.stderr)
        return 2
    if args.lookahead and (not cfg.mode.startswith("forecast") or args.path != "split" or cfg.ordered):
        print("--lookahead needs a forecast workload on the two-call path (--path split): "
              "only a forecast is known before the layer's own query", file=sys.stderr)
        return 2
    g = gpu_leg(args, cfg)
    ms_per_step = g["total_ms"] / args.steps
    if g["lookahead"] is not None:
        g["metrics"]["one_stream_ms_per_step"] = round(ms_per_step, 5)
        g["metrics"]["lookahead"] = g["lookahead"]["schedule"]
        ms_per_step = g["lookahead"]["ms_per_step"]
    value = cfg.batch / (ms_per_step / 1e3)
    # a step of one kernel: its duration is the timed region's (HIP events
    # around the K launches on their stream) divided by K; a step of two
    # kernels is split by the event pass
    if g["fused"]:
        kernels = {"step": {"ms": ms_per_step, "bytes": g["sel_bytes"] + g["dec_bytes"]}}
    elif g["dense"]:
        kernels = {"decode": {"ms": ms_per_step, "bytes": g["dec_bytes"]}}
    else:
        kernels = {
            "select": {"ms": g["sel_ms"], "bytes": g["sel_bytes"]},
            "decode": {"ms": g["dec_ms"], "bytes": g["dec_bytes"]},
        }
    for k in kernels.values():
        k["GB/s"] = k["bytes"] / (k["ms"] / 1e3) / 1e9
        k["frac"] = k["GB/s"] / HBM_PEAK_GBS
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dk = kernels[dom]
    workload = cfg.name + ("-dense" if g["dense"] else "")
    traffic = traffic_from_profiles(workload, dom)
    step_bytes = g["sel_bytes"] + g["dec_bytes"]
    kernel_ms = sum(v["ms"] for v in kernels.values())
    line = {
        "metric": "sparse decode tokens/s + achieved HBM GB/s (% of peak) at 32K-128K ctx, 1 GPU",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload, "batch": cfg.batch, "context": cfg.context,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "k": cfg.k, "k_e": cfg.k_e, "mode": cfg.mode,
                   "ordered": cfg.ordered, "tau": cfg.tau,
                   "path": "fused" if g["fused"] else ("dense" if g["dense"] else "split"),
                   "decode_steps_cycled": cfg.steps, "layer_instances": g["R"],
                   "timed_as": "one HIP graph of the K steps" if g["graph"] else "K launches",
                   "schedule": "lookahead, two streams" if g["lookahead"] else "one stream",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dk["GB/s"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dk["frac"], 4),
                     "traffic": traffic},
        "step_hbm": {"bytes": step_bytes, "GB/s": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernels": {k: {"ms": round(v["ms"], 5), "bytes": v["bytes"], "GB/s": round(v["GB/s"], 1),
                        "frac": round(v["frac"], 4)} for k, v in kernels.items()},
        "event_pass_ms": {"first": round(g["sel_ms"], 5), "second": round(g["dec_ms"], 5),
                          "note": "launches one by one with an event between kernels"},
        "launch_gap_us": round((ms_per_step - kernel_ms) * 1e3, 2),
        "metrics": g["metrics"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_leg(args, cfg)
    print(json.dumps(line), flush=True)
    return 0


# ----------------------------------------------------------------------------
# S2O prefill: one step = nsa_s2o_index + nsa_s2o_attend over one batch of
# prompts (every token's K/V already in the pools)
# ----------------------------------------------------------------------------
def prefill_flops(cfg, seq_lens, num_tiles) -> float:
    """Matrix-core flops the method needs for the walked tiles: 4 * D per
    (query, attended token) -- Q K^T and P V, two flops per multiply-add --
    over pass 1 (tokens [a, p] for the query at p) and the n* history tiles
    of its query tile (64 tokens each)."""
    import numpy as np
    seg, D = cfg.segment, cfg.head_dim
    pairs = 0
    for b, L in enumerate(seq_lens):
        for s in range(-(-int(L) // seg)):
            a = s * seg
            n = min(seg, int(L) - a)
            offs = np.arange(n)
            pairs += cfg.num_q_heads * int((offs + 1).sum())   # pass 1, every head
            nt = num_tiles[b, :, s, :-(-n // 64)].astype(np.int64)     # [Hq][tiles]
            sizes = np.minimum(64, n - 64 * np.arange(nt.shape[1]))
            pairs += int((nt * 64 * sizes[None, :]).sum())
    return 4.0 * D * pairs


def prefill_gpu_leg(args, cfg):
    import numpy as np
    import torch

    import workloads as W
    import block_sparse_kv_nsa_amd as N

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    pb = W.build_prefill(cfg)
    print(f"[bench] {cfg.name}: inputs drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    B, Hq, Hkv, D, seg = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.segment
    max_len = -(-cfg.seq_len // 64) * 64
    nseg = -(-max_len // seg)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q_host = np.zeros((B, Hq, max_len, D), dtype=np.uint16)
    q_host[:, :, :cfg.seq_len] = pb.q
    q, kp, vp = bf16(q_host), bf16(pb.k_pool), bf16(pb.v_pool)
    del q_host
    table = torch.from_numpy(pb.table).to(dev)
    lens = torch.from_numpy(pb.seq_lens).to(dev)
    shape = N.Shape.make(B, Hq, Hkv, D, cfg.max_blocks, cfg.num_phys_blocks, N.NSA_BF16)
    params = N.PrefillParams(seg, max_len, cfg.tau)
    ws_bytes = N.nsa_s2o_workspace_bytes(shape, params)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    q_perm = torch.empty((B, Hq, nseg, seg), dtype=torch.int32, device=dev)
    kv_perm = torch.empty((B, Hq, nseg, max_len), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, max_len, D), dtype=torch.bfloat16, device=dev)
    num_tiles = torch.empty((B, Hq, nseg, seg // 64), dtype=torch.int32, device=dev)

    def index():
        N.nsa_s2o_index(shape, params, q, kp, table, lens, q_perm, kv_perm, ws, ws_bytes)

    def attend():
        N.nsa_s2o_attend(shape, params, q, kp, vp, table, lens, q_perm, kv_perm, out, num_tiles,
                         ws, ws_bytes)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        index()
        if ev is not None:
            ev[1].record()
        attend()
        if ev is not None:
            ev[2].record()

    step()
    torch.cuda.synchronize()
    t_set = time.perf_counter()
    while time.perf_counter() - t_set < 0.25:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(1_000_000)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    n_ev = min(args.steps, 200)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for i in range(n_ev):
        step(evs[i])
    torch.cuda.synchronize()
    idx_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ev
    att_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / n_ev
    nt = num_tiles.cpu().numpy()
    flops = prefill_flops(cfg, pb.seq_lens, nt)
    walked, hist = 0, 0
    per_tile, full = [], 0
    for b, L in enumerate(pb.seq_lens):
        for s in range(-(-int(L) // seg)):
            n = min(seg, int(L) - s * seg)
            t = nt[b, :, s, :-(-n // 64)]
            walked += int(t.sum())
            hist += t.size * (s * seg // 64)
            if s:
                per_tile.append(t.flatten())
                full += int((t == s * seg // 64).sum())
    per_tile = np.concatenate(per_tile) if per_tile else np.zeros(1)
    walk_stats = {"mean": round(float(per_tile.mean()), 2),
                  "p50": int(np.percentile(per_tile, 50)), "p99": int(np.percentile(per_tile, 99)),
                  "max": int(per_tile.max()), "query_tiles_without_stop": full,
                  "query_tiles": int(per_tile.size)}
    dense_pairs = sum(Hq * int(L) * (int(L) + 1) // 2 for L in pb.seq_lens)
    return dict(total_ms=total_ms, wall_s=wall, idx_ms=idx_ms, att_ms=att_ms, flops=flops,
                walked=walked, hist=hist, dense_flops=4.0 * D * dense_pairs, walk_stats=walk_stats,
                ws_bytes=ws_bytes, tokens=int(sum(int(L) for L in pb.seq_lens)))


def prefill_cpu_leg(args, cfg):
    """The S2O oracle on a bounded sample of one (sequence, head): both orders
    of two segments (a quarter and three quarters in: a segment's cost grows
    about linearly with its history, so their mean stands for the mean
    segment) and four of their query tiles, scaled to every tile, segment,
    head and sequence."""
    import numpy as np

    import workloads as W
    from oracle import s2o_prefill as S

    host_cpus = os.cpu_count() or 1
    threads = min(host_cpus, 16)
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        limiter = None
    f = lambda a: W.stored_to_f64(a, cfg.dtype)  # noqa: E731
    keys, vals = (f(x) for x in W.kv_row(cfg, 0, 0))
    q = f(W.q_row(cfg, 0, 0))
    L, seg = q.shape[0], cfg.segment
    nseg = -(-L // seg)
    picks = sorted(set(int(round(x * (nseg - 1))) for x in (0.25, 0.75)))
    scale = 1.0 / math.sqrt(cfg.head_dim)
    tiles_per_seg = -(-seg // S.TILE)
    tile_pick = sorted(set(int(round(x)) for x in np.linspace(0, tiles_per_seg - 1, 4)))

    def one_segment(s):
        a, e = s * seg, min(s * seg + seg, L)
        t0 = time.perf_counter()
        qo, _ = S.query_order(q[a:e], keys, a, cfg.dtype)
        ko, _ = S.history_order(q[a:e], keys, a, cfg.dtype)
        t_orders = time.perf_counter() - t0
        t0 = time.perf_counter()
        for j in tile_pick:
            pos = a + qo[S.TILE * j:S.TILE * (j + 1)]
            S.query_tile(q[pos], pos, keys, vals, a, ko, cfg.tau, scale)
        return t_orders + (time.perf_counter() - t0) * tiles_per_seg / len(tile_pick)

    one_segment(1)                              # warm-up
    times = [sum(one_segment(s) for s in picks) for _ in range(3)]
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    per_pass = sorted(times)[1]
    step_s = per_pass / len(picks) * nseg * cfg.num_q_heads * cfg.batch
    return {"value": cfg.batch * cfg.seq_len / step_s, "unit": "tokens/s", "cores": threads,
            "host_cpus": host_cpus, "kind": "oracle",
            "sample": f"median of 3 passes (after a warm-up on segment 1) over segments {picks} of "
                      f"{nseg} of sequence 0, query head 0: both orders and query tiles "
                      f"{tile_pick} of {tiles_per_seg} (float64 NumPy, BLAS limited to {threads} "
                      f"threads); scaled to every tile, {nseg} segments, {cfg.num_q_heads} heads "
                      f"and {cfg.batch} sequences"}


def prefill_main(args) -> int:
    import workloads as W
    cfg = W.prefill_config(args.workload)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    g = prefill_gpu_leg(args, cfg)
    ms_per_step = g["total_ms"] / args.steps
    att_tflops = g["flops"] / (g["att_ms"] / 1e3) / 1e12
    kernels = {"index": {"ms": round(g["idx_ms"], 5)},
               "attend": {"ms": round(g["att_ms"], 5), "flops": g["flops"],
                          "TFLOP/s": round(att_tflops, 1),
                          "frac": round(att_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}}
    dom = "attend" if g["att_ms"] >= g["idx_ms"] else "index"
    line = {
        "metric": "S2O prefill tokens/s (segment orders + two-pass attention with early stop), 1 GPU",
        "value": round(g["tokens"] / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seq_len,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "segment": cfg.segment, "tau": cfg.tau,
                   "timed_as": "K x (nsa_s2o_index + nsa_s2o_attend)", "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": "attend", "achieved": kernels["attend"]["TFLOP/s"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": kernels["attend"]["frac"], "traffic": None},
        "dominant": dom,
        "kernels": kernels,
        "metrics": {"history_tiles_walked": g["walked"], "history_tiles": g["hist"],
                    "walk_per_query_tile": g["walk_stats"],
                    "density_vs_dense_causal": round(g["flops"] / g["dense_flops"], 4),
                    "workspace_bytes": g["ws_bytes"]},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = prefill_cpu_leg(args, cfg)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
