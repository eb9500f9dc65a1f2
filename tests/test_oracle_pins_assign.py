"""Pins for the communication-aware task assignment of the CPU oracle.

"Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
Training", Section 3.3: experts with a replica on the token's source node run
there; the others get the fewest remote nodes covering them (a minimum set
cover over remote-node bitmasks), then a random covering node each and a
uniform replica rank inside that node.  Pinned against an itertools brute
force of the set cover, validity of every assignment, closed forms for no
replication and for full replication, and the mapping of draws to choices.
"""
import itertools

import numpy as np
import pytest

import moe_inputs as mi
import oracle


def _nodes_of(holds, N):
    G, E = holds.shape
    per = G // N
    return [{r // per for r in np.nonzero(holds[:, e])[0]} for e in range(E)]


def brute_cover(experts, sn, nodes_of, N):
    """(size, value) smallest cover of the experts not on node sn, by trying
    node subsets of increasing size in itertools order."""
    need = [nodes_of[e] - {sn} for e in experts if sn not in nodes_of[e]]
    if not need:
        return 0
    remote = [n for n in range(N) if n != sn]
    for size in range(1, N):
        hits = [sum(1 << n for n in c)
                for c in itertools.combinations(remote, size)
                if all(set(c) & s for s in need)]
        if hits:
            return min(hits)
    raise AssertionError("no cover")


def _case(w, rho, seed):
    d = mi.make_inputs(w, seed=seed, with_x=False)
    idx, _ = oracle.gate(d["logits"], w.K)
    holds = mi.replica_layout(w.E, w.R, rho, seed)
    rng = np.random.Generator(np.random.PCG64(seed + 100))
    src = rng.integers(0, w.R, w.T).astype(np.int32)
    un, ur = mi.assign_draws(w.T, w.K, seed)
    return idx, holds, src, un, ur


SHAPES = [mi.DEEPSEEK_V3.replace(T=96), mi.QWEN3.replace(T=96),
          mi.KIMI.replace(T=24), mi.TINY]


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("rho", [0.0, 0.5, 1.0])
def test_assignment_is_a_minimum_cover_and_valid(w, rho):
    idx, holds, src, un, ur = _case(w, rho, 1)
    ar, rm = oracle.assign(idx, src, holds, w.N, un, ur)
    nodes_of = _nodes_of(holds, w.N)
    per = w.R // w.N
    for t in range(w.T):
        sn = src[t] // per
        assert int(rm[t]) == brute_cover(idx[t], sn, nodes_of, w.N)
        b = {n for n in range(w.N) if (int(rm[t]) >> n) & 1}
        for k in range(w.K):
            e, r = idx[t, k], ar[t, k]
            assert holds[r, e] == 1                      # a real replica
            node = r // per
            if sn in nodes_of[e]:
                assert node == sn                        # local experts stay
            else:
                assert node in b and node in nodes_of[e]


def test_no_replication_reduces_to_the_static_placement():
    w = mi.DEEPSEEK_V3.replace(T=64)
    idx, _, src, un, ur = _case(w, 0.0, 2)
    holds = mi.replica_layout(w.E, w.R, 0.0, 2)
    ar, rm = oracle.assign(idx, src, holds, w.N, un, ur)
    per_rank, per_node = w.E // w.R, w.R // w.N
    np.testing.assert_array_equal(ar, idx // per_rank)
    home = (idx // per_rank) // per_node
    sn = src // per_node
    want = [sum(1 << int(n) for n in set(home[t]) - {sn[t]})
            for t in range(w.T)]
    np.testing.assert_array_equal(rm.astype(np.int64), want)


def test_full_replication_stays_on_the_source_node():
    T, E, K, G, N = 32, 16, 4, 8, 4
    idx = mi.random_topk_idx(T, E, K, seed=3)
    holds = np.zeros((G, E), np.uint8)
    holds[0::2] = 1                                  # every node: rank 2n
    src = (np.arange(T) % G).astype(np.int32)
    un, ur = mi.assign_draws(T, K, 3)
    ar, rm = oracle.assign(idx, src, holds, N, un, ur)
    assert not rm.any()
    np.testing.assert_array_equal(ar, np.repeat((src // 2 * 2)[:, None], K,
                                                axis=1))


def test_draws_pick_the_floor_of_u_times_count():
    # expert 0 on ranks 0, 1, 3 of node 0 (4 ranks a node); source node 0
    G, N, E = 8, 2, 2
    holds = np.zeros((G, E), np.uint8)
    holds[[0, 1, 3], 0] = 1
    holds[4, 1] = 1
    idx = np.zeros((3, 1), np.int32)
    src = np.zeros(3, np.int32)
    # u = (2j+1) * 2^32 / 6 lands inside candidate j of 3
    ur = np.array([[(2 * j + 1) * (1 << 32) // 6] for j in range(3)], np.uint32)
    ar, _ = oracle.assign(idx, src, holds, N, ur, ur)
    np.testing.assert_array_equal(ar.ravel(), [0, 1, 3])
    # remote node choice: expert 1 only on node 1 rank 4; expert 0 on both
    holds2 = holds.copy()
    holds2[6, 0] = 1
    idx2 = np.array([[1, 0]], np.int32)
    src2 = np.array([0], np.int32)
    ar2, rm2 = oracle.assign(idx2, src2, holds2, N,
                             np.zeros((1, 2), np.uint32),
                             np.zeros((1, 2), np.uint32))
    assert int(rm2[0]) == 0b10 and ar2[0, 0] == 4 and ar2[0, 1] == 0


def test_cover_prefers_fewer_nodes_then_lower_mask():
    # experts A on nodes {1,2}, B on {2,3}, C on {1,3}: any two nodes cover;
    # the lowest two-node mask is {1,2} = 0b0110
    G, N, E = 4, 4, 3
    holds = np.zeros((G, E), np.uint8)
    holds[[1, 2], 0] = 1
    holds[[2, 3], 1] = 1
    holds[[1, 3], 2] = 1
    idx = np.array([[0, 1, 2]], np.int32)
    ar, rm = oracle.assign(idx, np.array([0], np.int32), holds, N,
                           np.zeros((1, 3), np.uint32),
                           np.zeros((1, 3), np.uint32))
    assert int(rm[0]) == 0b0110
    # B's candidates within {1,2} are {2}; C's are {1}
    np.testing.assert_array_equal(ar[0], [1, 2, 1])
