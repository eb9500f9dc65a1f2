"""The allocation-free fused call, moe_dispatch_combine_noalloc, against the
fused call with a caller workspace (moe_dispatch_combine): both run the same
kernels, so every output must be bit-identical.  Calls follow one another on
one GPU with shrinking inputs, so each reuses the static scratch the previous
one left behind."""
import ctypes

import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
from helpers import (LAYOUT_KEYS, cfg_of, dev, host, layout_to_host,
                     out_dtype, require_gpu, row_dtype)


def _buffers(w):
    cfg = cfg_of(w)
    T, K = w.T, w.K
    return dict(
        cfg=cfg,
        idx=torch.full((T * K,), -7, dtype=torch.int32, device="cuda"),
        wt=torch.full((T * K,), -7.0, dtype=torch.float32, device="cuda"),
        lay=moe.alloc_layout(cfg),
        send=torch.zeros((T * K, w.H), dtype=row_dtype(w), device="cuda"),
        out=torch.zeros((T, w.H), dtype=out_dtype(w), device="cuda"))


def _host(w, b):
    res = layout_to_host(b["lay"], w.T, w.K, w.N)
    res.update(topk_idx=host(b["idx"]), topk_w=host(b["wt"]),
               send=host(b["send"]), out=host(b["out"]))
    return res


@pytest.mark.gpu
def test_noalloc_matches_fused_call_with_shrinking_inputs():
    require_gpu()
    cases = [mi.DEEPSEEK_V3.replace(T=5000, H=512),   # 79 tiles; the gate
                                                      # writes the counts
             mi.KIMI.replace(T=2000, H=256),          # larger E, fewer tokens
             mi.DEEPSEEK_V3_DECODE]                   # the decode launch
    inputs = [mi.make_inputs(w) for w in cases]
    dev_in = [(dev(d["x"]), dev(d["logits"]), dev(d["expert_scale"]))
              for d in inputs]
    # the allocation-free calls first, back to back on one stream
    got = []
    for w, (x, lg, sc) in zip(cases, dev_in):
        print(f"noalloc: {w.name} T={w.T} H={w.H} E={w.E} K={w.K}",
              flush=True)
        b = _buffers(w)
        moe.moe_dispatch_combine_noalloc(b["cfg"], x, lg, sc, b["idx"],
                                         b["wt"], b["lay"], b["send"],
                                         b["out"])
        got.append(b)
    torch.cuda.synchronize()
    # then the same inputs through the call with a caller workspace
    for w, (x, lg, sc), b in zip(cases, dev_in, got):
        r = _buffers(w)
        ws = moe.alloc_workspace(r["cfg"])
        moe.moe_dispatch_combine(r["cfg"], x, lg, sc, r["idx"], r["wt"],
                                 r["lay"], r["send"], r["out"], ws)
        assert moe.moe_read_device_error(ws) == 0
        a, c = _host(w, b), _host(w, r)
        for k in LAYOUT_KEYS + ("topk_idx", "topk_w", "send", "out"):
            np.testing.assert_array_equal(a[k], c[k], err_msg=f"{w.name} {k}")


@pytest.mark.gpu
def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    require_gpu()
    # E = 4096 takes 64-token layout tiles: 5000 tokens need about 1.3 MiB
    w = mi.Workload("big", T=5000, H=8, E=4096, K=8, R=64, N=8)
    b = _buffers(w)
    assert moe.moe_workspace_bytes(b["cfg"]) > moe.MOE_SCRATCH_BYTES
    d = mi.make_inputs(w)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_dispatch_combine_noalloc(b["cfg"], dev(d["x"]),
                                         dev(d["logits"]), None, b["idx"],
                                         b["wt"], b["lay"], b["send"],
                                         b["out"])
    assert ei.value.code == moe.MOE_ESCRATCH
    torch.cuda.synchronize()
    assert bool((b["idx"] == -7).all()) and not bool(b["out"].any())


def test_noalloc_scratch_limit_checked_on_host():
    # returns before any HIP call: the pointers below are never dereferenced
    lib = moe.lib()
    big = moe.make_cfg(T=5000, H=8, E=4096, K=8, R=64, N=8)
    ok = moe.make_cfg(T=3904, H=8, E=4096, K=8, R=64, N=8)
    assert moe.moe_workspace_bytes(big) > moe.MOE_SCRATCH_BYTES
    assert moe.moe_workspace_bytes(ok) <= moe.MOE_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    lay = moe.moe_layout(*([fake.value] * 11))
    rc = lib.moe_dispatch_combine_noalloc(ctypes.byref(big), fake, fake, None,
                                          fake, fake, ctypes.byref(lay), fake,
                                          fake, None)
    assert rc == moe.MOE_ESCRATCH
    assert "scratch" in moe.moe_strerror(rc)
    assert lib.moe_dispatch_combine_noalloc(
        ctypes.byref(big), None, None, None, None, None, ctypes.byref(lay),
        None, None, None) == moe.MOE_EINVAL
