"""GPU parity of the communication-aware task assignment (integer and bitmask
work: bit-exact against the CPU oracle)."""
import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
import oracle
from helpers import cfg_of, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _case(w, rho, seed, src_kind="random"):
    d = mi.make_inputs(w, seed=seed, with_x=False)
    idx, _ = oracle.gate(d["logits"], w.K)
    holds = mi.replica_layout(w.E, w.R, rho, seed)
    if src_kind == "random":
        rng = np.random.Generator(np.random.PCG64(seed + 7))
        src = rng.integers(0, w.R, w.T).astype(np.int32)
    else:
        src = np.zeros(w.T, np.int32)
    un, ur = mi.assign_draws(w.T, w.K, seed)
    return idx, holds, src, un, ur


def gpu_assign(w, idx, holds, src, un, ur):
    cfg = cfg_of(w)
    ar = torch.empty(w.T * w.K, dtype=torch.int32, device="cuda")
    rm = torch.empty(w.T, dtype=torch.int64, device="cuda")
    ws = moe.alloc_assign_workspace(cfg)
    moe.moe_assign_tasks(cfg, dev(idx), dev(src), dev(holds),
                         dev(un.view(np.int32)), dev(ur.view(np.int32)), ar,
                         rm, ws)
    err = moe.moe_read_device_error(ws)
    return host(ar).reshape(w.T, w.K), host(rm).view(np.uint64), err


SHAPES = [mi.TINY, mi.MIXTRAL.replace(T=500), mi.QWEN3.replace(T=1000),
          mi.DEEPSEEK_V3.replace(T=2000), mi.KIMI.replace(T=300)]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("rho", [0.0, 0.5, 1.0])
def test_assign(w, rho):
    idx, holds, src, un, ur = _case(w, rho, 1)
    ar, rm, err = gpu_assign(w, idx, holds, src, un, ur)
    assert err == 0
    rar, rrm = oracle.assign(idx, src, holds, w.N, un, ur)
    np.testing.assert_array_equal(rm, rrm)
    np.testing.assert_array_equal(ar, rar)


def test_assign_full_size_deepseek():
    w = mi.DEEPSEEK_V3
    idx, holds, src, un, ur = _case(w, 0.5, 0, src_kind="zero")
    ar, rm, err = gpu_assign(w, idx, holds, src, un, ur)
    assert err == 0
    rar, rrm = oracle.assign(idx, src, holds, w.N, un, ur)
    np.testing.assert_array_equal(rm, rrm)
    np.testing.assert_array_equal(ar, rar)


def test_assign_full_size_kimi_sampled():
    w = mi.KIMI
    idx, holds, src, un, ur = _case(w, 0.5, 0)
    ar, rm, err = gpu_assign(w, idx, holds, src, un, ur)
    assert err == 0
    rng = np.random.Generator(np.random.PCG64(2))
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.integers(0, w.T, 254)]))
    rar, rrm = oracle.assign(idx[toks], src[toks], holds, w.N, un[toks],
                             ur[toks])
    np.testing.assert_array_equal(rm[toks], rrm)
    np.testing.assert_array_equal(ar[toks], rar)


def test_assign_device_errors():
    w = mi.DEEPSEEK_V3.replace(T=64)
    idx, holds, src, un, ur = _case(w, 0.0, 3)
    holds = holds.copy()
    holds[:, 5] = 0                              # expert 5 has no replica
    idx[0, 0] = 5 if 5 not in idx[0] else idx[0, 0]
    src[1] = w.R + 3                             # bad source rank
    ar, rm, err = gpu_assign(w, idx, holds, src, un, ur)
    assert err & moe.MOE_DEVERR_SRC_RANK
    assert np.all(ar[1] == -1)
    bad_tok = np.nonzero((idx == 5).any(axis=1))[0]
    assert len(bad_tok) and err & moe.MOE_DEVERR_NO_REPLICA
    assert np.all(ar[bad_tok] == -1)
    ok = np.setdiff1d(np.arange(w.T), np.concatenate([bad_tok, [1]]))
    rar, rrm = oracle.assign(idx[ok], src[ok], holds, w.N, un[ok], ur[ok])
    np.testing.assert_array_equal(ar[ok], rar)
    np.testing.assert_array_equal(rm[ok], rrm)


def test_assign_both_cover_searches():
    # 16 nodes and about 3 replicas per expert: about half of the tokens
    # have more than 12 candidate nodes (the wave walks subsets in order),
    # the rest at most 12 (the wave tests all subsets at once)
    w = mi.Workload("cover", T=300, H=8, E=96, K=16, R=32, N=16)
    holds = mi.replica_layout(w.E, w.R, 2.0, 3)
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=3)
    rng = np.random.Generator(np.random.PCG64(4))
    src = rng.integers(0, w.R, w.T).astype(np.int32)
    un, ur = mi.assign_draws(w.T, w.K, 3)
    ar, rm, err = gpu_assign(w, idx, holds, src, un, ur)
    assert err == 0
    rar, rrm = oracle.assign(idx, src, holds, w.N, un, ur)
    np.testing.assert_array_equal(rm, rrm)
    np.testing.assert_array_equal(ar, rar)
    # both searches ran: count candidate nodes per token on the host
    per_node = w.R // w.N
    nodes_of = [set((np.nonzero(holds[:, e])[0] // per_node).tolist())
                for e in range(w.E)]
    big = 0
    for t in range(w.T):
        sn = int(src[t]) // per_node
        rem = [nodes_of[e] - {sn} for e in idx[t] if sn not in nodes_of[e]]
        forced = set().union(*[r for r in rem if len(r) == 1]) if rem else set()
        uni = set().union(*[r for r in rem if not (r & forced)] or [set()])
        big += len(uni) > 12
    assert 0 < big < w.T
