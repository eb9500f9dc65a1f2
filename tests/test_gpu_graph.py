"""HIP graph capture of the fused paths: every replay equals the eager run.

The library enqueues kernel launches only (no memsets, allocations or
synchronisation inside a call), so a whole step can be captured and
replayed.  Each test runs the path eagerly, captures it, then replays it
several times with eager work in between (outputs cleared by the program's
own fill kernels) and checks every replay against the eager result bit for
bit (the path is deterministic).
"""
import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
from helpers import cfg_of, dev, out_dtype, require_gpu, row_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _replays_match(step, outs, n=3):
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(n):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ww in zip(outs, want):
            assert torch.equal(o, ww)


@pytest.mark.parametrize("w", [mi.DEEPSEEK_V3_DECODE,
                               mi.QWEN3.replace(T=1000, H=512)],
                         ids=lambda w: w.name)
def test_graph_flat(w):
    d = mi.make_inputs(w)
    cfg = cfg_of(w)
    x, lg = dev(d["x"]), dev(d["logits"])
    sc = dev(d["expert_scale"])
    idx = torch.empty(w.T * w.K, dtype=torch.int32, device="cuda")
    wt = torch.empty(w.T * w.K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg)
    send = torch.empty((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)

    def step():
        moe.moe_dispatch_combine(cfg, x, lg, sc, idx, wt, lay, send, out, ws)

    _replays_match(step, [idx, wt, lay.slot_pos, lay.row_src, lay.node_slot,
                          send, out])
    assert moe.moe_read_device_error(ws) == 0


def test_graph_fp8_and_two_leg():
    w = mi.DEEPSEEK_V3.replace(T=300, H=512)
    d = mi.make_inputs(w)
    cfg = cfg_of(w)
    x, lg = dev(d["x"]), dev(d["logits"])
    sc = dev(d["expert_scale"])
    idx = torch.empty(w.T * w.K, dtype=torch.int32, device="cuda")
    wt = torch.empty(w.T * w.K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg)
    rb = moe.moe_fp8_row_bytes(w.H, 128)
    send8 = torch.empty((w.T * w.K, rb), dtype=torch.uint8, device="cuda")
    cap = moe.moe_node_rows_max(cfg)
    ns = torch.empty((cap, w.H), dtype=row_dtype(w), device="cuda")
    send = torch.empty((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    part = torch.empty((cap, w.H), dtype=torch.bfloat16, device="cuda")
    out8 = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    out2 = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)

    def step():
        moe.moe_dispatch_combine_fp8(cfg, x, lg, sc, idx, wt, lay, send8,
                                     out8, ws)
        moe.moe_dispatch_combine_nodes(cfg, x, lg, sc, idx, wt, lay, ns, send,
                                       part, out2, ws)

    _replays_match(step, [send8, out8, send, out2])
