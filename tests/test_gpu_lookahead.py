"""SparDA's lookahead (SparDA summary, "Trainierbare Lookahead Sparse-Selektion"):
the forecast made in layer l selects layer l+1's blocks, so layer l+1's
selection can run on a second stream while layer l decodes.  A stack of
layers run on that two-stream schedule gives the same selections and the
same output bits as the same layers run one after the other on one stream,
and the selections agree with the oracle.
"""

from __future__ import annotations

import pytest
import torch

import workloads as W
from tests import gpu_harness as H

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LAYERS = 4
TOKENS = 3


def _stack():
    cfgs = [W.Config(f"lookahead-{l}", 80 + l, batch=3, context=64 * 90 + 17, num_q_heads=8,
                     num_kv_heads=2, head_dim=128, dtype="bf16", mode="forecast", k=12, k_e=0,
                     steps=TOKENS) for l in range(LAYERS)]
    layers = []
    for cfg in cfgs:
        lay = H.make_layer(cfg, W.build_batch(cfg))
        H.prefill(lay, cfg)
        layers.append(lay)
    dev = layers[0].device
    lens = [torch.full((cfgs[0].batch,), cfgs[0].seq_len(t), dtype=torch.int32, device=dev)
            for t in range(TOKENS)]
    fcs = [H.device_query(cfg, 0) for cfg in cfgs]
    qs = [[H.device_q(cfg, t) for t in range(TOKENS)] for cfg in cfgs]
    return cfgs, layers, lens, fcs, qs


def _record(lay, outs):
    """Copies of a layer's results, taken on the current stream right after
    its decode (before the layer's next selection can overwrite them)."""
    outs.append((lay.selected.clone(), lay.num_selected.clone(), lay.out.clone()))


def test_lookahead_schedule_matches_one_stream():
    H.log(f"[case] lookahead: {LAYERS} forecast layers, {TOKENS} tokens, two streams vs one")
    cfgs, layers, lens, fcs, qs = _stack()
    assert all(cfgs[0].seq_len(t) % 64 != 0 for t in range(TOKENS))
    L = [cfgs[0].seq_len(t) for t in range(TOKENS)]

    # one stream: select then decode, layer by layer
    want = []
    for t in range(TOKENS):
        for l, lay in enumerate(layers):
            lay.seq_lens = lens[t]
            lay.select(fcs[l], L[t])
            lay.decode(qs[l][t])
            _record(lay, want)
    torch.cuda.synchronize()

    # two streams: step i = (token i // LAYERS, layer i % LAYERS); the
    # selection of step i+1 waits for step i-1's decode, the decode of step i
    # for its own selection
    cfgs, layers, lens, fcs, qs = _stack()
    sel_stream = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    n = TOKENS * LAYERS
    sel_done = [torch.cuda.Event() for _ in range(n)]
    dec_done = [torch.cuda.Event() for _ in range(n)]

    def select(i):
        t, l = divmod(i, LAYERS)
        layers[l].seq_lens = lens[t]
        layers[l].select(fcs[l], L[t], stream=sel_stream.cuda_stream)
        sel_done[i].record(sel_stream)

    got = []
    select(0)
    for i in range(n):
        t, l = divmod(i, LAYERS)
        if i + 1 < n:
            if i > 0:
                sel_stream.wait_event(dec_done[i - 1])
            select(i + 1)
        main.wait_event(sel_done[i])
        layers[l].decode(qs[l][t], stream=main.cuda_stream)
        _record(layers[l], got)
        dec_done[i].record(main)
    torch.cuda.synchronize()

    assert len(got) == len(want)
    for (s1, n1, o1), (s2, n2, o2) in zip(want, got):
        assert torch.equal(n1, n2)
        assert torch.equal(s1, s2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))

    # the last token of every layer against the oracle
    for cfg, lay in zip(cfgs, layers):
        res = H.fetch(lay)
        for b in range(cfg.batch):
            for g in range(cfg.num_kv_heads):
                H.check_step(cfg, res, H.oracle_row(cfg, b, g), b, g, TOKENS - 1)
