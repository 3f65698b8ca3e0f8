"""Run in a child process by test_gpu_checks.py, with NSA_LIB_PATH naming the
library built with the device-side contract checks: each case breaks one
item of the caller's contract, runs one call and prints the bits the
library recorded.  Every broken value is one the checks clamp before any
access; the script refuses to launch anything on a library without them."""

from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import block_sparse_kv_nsa_amd as N  # noqa: E402
import workloads as W  # noqa: E402
from tests import gpu_harness as H  # noqa: E402


def main() -> int:
    if not N.nsa_debug_checks():
        print("REFUSED: library without device checks", flush=True)
        return 3
    torch.cuda.set_device(0)
    cfg = W.Config("checks", 90, batch=2, context=64 * 30 + 9, num_q_heads=8, num_kv_heads=2,
                   head_dim=128, dtype="bf16", mode="group_softmax", k=12, k_e=8, steps=1)
    batch = W.build_batch(cfg)
    L = cfg.seq_len(0)
    nb = L // 64
    results = {}

    def fresh():
        layer = H.make_layer(cfg, batch)
        H.prefill(layer, cfg)
        layer.seq_lens.fill_(L)
        torch.cuda.synchronize()
        N.nsa_debug_error(True)
        return layer

    def run(name, layer, fused):
        print(f"[case] {name}", flush=True)
        if fused:
            layer.step(H.device_query(cfg, 0), H.device_q(cfg, 0), L)
        else:
            layer.select(H.device_query(cfg, 0), L)
            layer.decode(H.device_q(cfg, 0))
        torch.cuda.synchronize()
        results[name] = N.nsa_debug_error(True)

    layer = fresh()
    run("clean two calls", layer, False)
    layer = fresh()
    run("clean fused", layer, True)
    # the tail block's table entry past the pool (both paths read it)
    for fused in (False, True):
        layer = fresh()
        layer.block_table[1, nb] = cfg.num_phys_blocks + 7
        run(f"table entry {'fused' if fused else 'two calls'}", layer, fused)
    # a listed block id past the row's full blocks (decode)
    layer = fresh()
    layer.select(H.device_query(cfg, 0), L)
    torch.cuda.synchronize()
    layer.selected[0, 1, 0] = nb + 3
    print("[case] listed id", flush=True)
    layer.decode(H.device_q(cfg, 0))
    torch.cuda.synchronize()
    results["listed id"] = N.nsa_debug_error(True)
    # an eviction-set id past the row's full blocks (steady fused step)
    layer = fresh()
    layer.step(H.device_query(cfg, 0), H.device_q(cfg, 0), L)
    torch.cuda.synchronize()
    N.nsa_debug_error(True)
    layer.evict_set[1, 0, 0] = nb + 5
    run("eviction id fused", layer, True)
    # a sequence longer than its table row
    layer = fresh()
    layer.seq_lens[0] = 64 * cfg.max_blocks + 70
    print("[case] seq_len", flush=True)
    layer.select(H.device_query(cfg, 0), 64 * cfg.max_blocks)
    layer.decode(H.device_q(cfg, 0))
    torch.cuda.synchronize()
    results["seq_len"] = N.nsa_debug_error(True)
    for k, v in results.items():
        print(f"RESULT {k}: {v}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
