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
WORKLOADS = {"tiny-fp32": 0, "nosa-1b": 1, "sparda-8b": 2, "long-128k": 3, "early-stop": 4}
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
    ap.add_argument("--workload", default="long-128k", choices=sorted(WORKLOADS))
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
                         "nsa_sparse_decode")
    return ap.parse_args()


def source_hash(rel: str) -> str:
    h = hashlib.sha256()
    for part in (rel, "block_sparse_kv_nsa_amd/csrc/nsa_device.hpp",
                 "block_sparse_kv_nsa_amd/csrc/nsa_internal.hpp",
                 "block_sparse_kv_nsa_amd/csrc/nsa_attend.hpp"):
        with open(os.path.join(ROOT, part), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# algorithmic bytes: what the method must move per launch
# ----------------------------------------------------------------------------
def select_bytes(cfg, L: int) -> int:
    e = 2 if cfg.dtype == "bf16" else 4
    nb = L // 64
    reps = cfg.rows * nb * 4 * cfg.head_dim * e
    qv = (cfg.batch * cfg.num_kv_heads if cfg.mode == "forecast" else cfg.batch * cfg.num_q_heads)
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

    kp, vp = to_dev(batch.k_pool), to_dev(batch.v_pool)
    table = torch.from_numpy(batch.table).to(dev)
    logits = torch.from_numpy(batch.logits).to(dev)
    pool_bytes = 2 * kp.numel() * kp.element_size()
    R = args.instances or max(2, min(16, math.ceil((1 << 30) / max(1, select_bytes(cfg, cfg.seq_len(0))
                                                                    + decode_bytes(cfg, cfg.seq_len(0), cfg.k)))))
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
    sel_q = ([to_dev(W.forecasts(cfg))] * steps) if cfg.mode == "forecast" else qs
    fills = [(cfg.seq_len(t) % 64) == 0 for t in range(steps)]
    fill_first = [torch.full((cfg.batch,), cfg.seq_len(t) // 64 - 1, dtype=torch.int32, device=dev)
                  for t in range(steps)]
    ones = torch.ones(cfg.batch, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    fused = args.path == "fused" and not cfg.ordered

    def step(i, ev=None):
        lay = layers[i % R]
        t = i % steps
        lay.seq_lens = lens[t]
        if fills[t]:
            lay.update_reps(fill_first[t], ones, 1, stream)
        if ev is not None:
            ev[0].record(stream)
        if fused:
            lay.step(sel_q[t], qs[t], cfg.seq_len(t), stream)
            if ev is not None:
                ev[1].record(stream)
                ev[2].record(stream)
            return
        lay.select(sel_q[t], cfg.seq_len(t), stream)
        if ev is not None:
            ev[1].record(stream)
        lay.decode(qs[t], stream)
        if ev is not None:
            ev[2].record(stream)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the K timed steps: nothing but the steps between the two events
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    # per-kernel durations: the same steps again with events around each launch
    # on the launch stream (an event between launches adds a small gap, so
    # this pass is kept apart from the timed one)
    n_ev = min(args.steps, 1000)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for i in range(n_ev):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    sel_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / n_ev
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / n_ev

    n_sel = layers[0].num_selected.float().mean().item()
    L_mid = cfg.seq_len(steps // 2)
    sb = select_bytes(cfg, L_mid)
    db = decode_bytes(cfg, L_mid, int(round(n_sel)))
    return dict(R=R, total_ms=total_ms, wall_s=wall, sel_ms=sel_ms, dec_ms=dec_ms,
                sel_bytes=sb, dec_bytes=db, n_sel=n_sel, fused=fused)


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ----------------------------------------------------------------------------
def cpu_leg(args, cfg):
    import numpy as np

    import workloads as W
    from oracle import nsa_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
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
        row.reps(cfg.nb0)
        if cfg.k_e:
            row.eviction_scores(cfg.nb0)
        qs = [W.stored_to_f64(W.query_row(cfg, b, g, t), cfg.dtype) for t in range(cfg.steps)]
        f = W.stored_to_f64(W.forecast_row(cfg, b, g), cfg.dtype) if cfg.mode == "forecast" else None
        sample.append((row, qs, f))
    # the workload's decode steps on the sampled rows, repeated until the
    # budget is spent (a repeated step does the same work: no block fills)
    spent, done, passes = 0.0, 0, 0
    while spent < args.cpu_seconds:
        for row, qs, f in sample:
            for t in range(cfg.steps):
                t0 = time.perf_counter()
                row.step(cfg.seq_len(t), qs[t], f=f)
                spent += time.perf_counter() - t0
                done += 1
        passes += 1
    per_row_step = spent / done
    step_s = per_row_step * cfg.rows
    return {"value": cfg.batch / step_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} row-steps ({passes} passes over the {cfg.steps} decode steps of "
                      f"{len(sample)} of {cfg.rows} rows; float64 NumPy, one row at a time), "
                      f"{spent:.1f}s timed; scaled to all rows"}


KERNEL_SYMBOLS = {"step": "gang_kernel", "select": "score_select_kernel", "decode": "decode_kernel"}
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
    kernel = "step" if args.path == "fused" else "select"
    kernels = [kernel] if args.path == "fused" else ["select", "decode"]
    for kern in kernels:
        sym = KERNEL_SYMBOLS[kern]
        f_k, w_k = pick(fetch, sym) * 1024, pick(write, sym) * 1024
        rec = {
            "kernel": kern, "symbol": sym, "workload": args.workload,
            "fetch_bytes_raw": f_k, "write_bytes_raw": w_k,
            "calibration": {"kernel": CALIBRATION_SYMBOL, "bytes_each_way": known,
                            "fetch_bytes_raw": f_cal, "write_bytes_raw": w_cal,
                            "fetch_scale": known / f_cal, "write_scale": known / w_cal},
            "bytes_per_launch": f_k * known / f_cal + w_k * known / w_cal,
            "source_hash": source_hash(KERNEL_SOURCES[kern]),
            "files": list(args.traffic_from),
        }
        path = os.path.join(ROOT, "profiles", f"{kern}_{args.workload}_traffic.json")
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
    import workloads as W
    cfg = W.config(WORKLOADS[args.workload])
    g = gpu_leg(args, cfg)
    ms_per_step = g["total_ms"] / args.steps
    value = cfg.batch / (ms_per_step / 1e3)
    if g["fused"]:
        kernels = {"step": {"ms": g["sel_ms"], "bytes": g["sel_bytes"] + g["dec_bytes"]}}
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
    traffic = traffic_from_profiles(args.workload, dom)
    step_bytes = g["sel_bytes"] + g["dec_bytes"]
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
        "config": {"workload": cfg.name, "batch": cfg.batch, "context": cfg.context,
                   "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "k": cfg.k, "k_e": cfg.k_e, "mode": cfg.mode,
                   "decode_steps_cycled": cfg.steps, "layer_instances": g["R"],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dk["GB/s"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dk["frac"], 4),
                     "traffic": traffic},
        "step_hbm": {"bytes": step_bytes, "GB/s": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernels": {k: {"ms": round(v["ms"], 5), "bytes": v["bytes"], "GB/s": round(v["GB/s"], 1),
                        "frac": round(v["frac"], 4)} for k, v in kernels.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_leg(args, cfg)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
