"""Seeded synthetic workloads for the MoE dispatch/combine path.

This module only *creates inputs*: workload shapes, gate logits, hidden rows
and the per-expert scale of the stand-in expert.  It holds none of the
method's arithmetic (no top-K, no layout, no packing, no combine), so both the
CPU oracle and the HIP library can be fed from it without sharing any code.

Every generator draws from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order: gate-logit noise ``[T, E]`` (fp32), then hidden rows ``x [T, H]``
(fp32, rounded to bf16 where the workload is bf16), then any per-token
cluster ids ``[T]``.  bf16 values are carried on the host as ``uint16`` bit
patterns.

Workload shapes follow the expert-parallel settings the pages discuss: the
Mixtral/DeepSeek-V3 model families named in "Efficient and portable
mixture-of-experts communication" ("Introdución"), DeepSeek-V3's 256 experts
with top-8 and 7,168-wide BF16 embeddings in "MoX: Efficient MoE Routing on
Direct-Connect Topologies" (Section 3, Methodology), and the skewed,
co-activated expert demand described in MoX (Section 1) and in "Cobalt:
Leveraging Expert Co-activation for Efficient Distributed MoE Training"
(Section 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic workload.

    T tokens, hidden size H, E experts, top-K, R logical EP ranks holding E/R
    contiguous experts each, N logical nodes holding R/N contiguous ranks each.
    """

    name: str
    T: int
    H: int
    E: int
    K: int
    R: int
    N: int
    x_dtype: str = BF16
    out_dtype: str = BF16
    # logit recipe: "normal", "zipf" (N(0,1) - s*ln(e+1)) or "clusters"
    logits: str = "normal"
    zipf_s: float = 0.0
    n_clusters: int = 0
    cluster_bias: float = 0.0
    # stand-in expert: "identity", "linear" (1+0.01*e), "mod8" (1+0.01*(e%8))
    expert: str = "mod8"
    renorm: bool = True
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.T * self.K

    @property
    def elem_bytes(self) -> int:
        return 4 if self.x_dtype == F32 else 2

    @property
    def out_elem_bytes(self) -> int:
        return 4 if self.out_dtype == F32 else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def algorithmic_bytes(self) -> int:
        """Bytes the whole path must move at least once.

        x read once, K packed rows written, K rows read back by the combine,
        one output row written, the fp32 logits, the per-(token, slot) routing
        metadata (index, weight, slot position, source row: 4 x 4 B, each
        written once and read once -> 32 B) plus the 8-byte node mask, and the
        per-expert/rank/node count and offset arrays.
        """
        b = self.elem_bytes
        ob = self.out_elem_bytes
        T, H, E, K = self.T, self.H, self.E, self.K
        per_token = (K + 1) * H * b + K * H * b + H * ob + 4 * E + 32 * K + 8
        return T * per_token + 8 * (E + self.R + self.N)


TINY = Workload("tiny", T=16, H=64, E=8, K=2, R=4, N=2, x_dtype=F32,
                out_dtype=F32, logits="normal", expert="identity")
MIXTRAL = Workload("mixtral", T=4096, H=4096, E=8, K=2, R=8, N=1,
                   logits="normal", expert="linear")
QWEN3 = Workload("qwen3_skewed", T=8192, H=2048, E=128, K=8, R=64, N=8,
                 logits="zipf", zipf_s=1.0, expert="mod8")
DEEPSEEK_V3 = Workload("deepseek_v3", T=16384, H=7168, E=256, K=8, R=64, N=8,
                       logits="clusters", n_clusters=16, cluster_bias=1.5,
                       expert="mod8")
DEEPSEEK_V3_DECODE = DEEPSEEK_V3.replace(name="deepseek_v3_decode", T=128)
KIMI = Workload("kimi", T=32768, H=7168, E=896, K=16, R=128, N=16,
                logits="zipf", zipf_s=1.2, expert="mod8")

WORKLOADS = {w.name: w for w in
             (TINY, MIXTRAL, QWEN3, DEEPSEEK_V3, DEEPSEEK_V3_DECODE, KIMI)}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.

    Used only to *create* bf16 inputs.  Inputs never hold NaN.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def expert_scale(w: Workload) -> Optional[np.ndarray]:
    """Per-expert factor s_e of the diagonal stand-in expert, fp32 [E].

    Computed in fp64 and rounded once to fp32.  ``None`` for identity experts.
    """
    e = np.arange(w.E, dtype=np.float64)
    if w.expert == "identity":
        return None
    if w.expert == "linear":
        return (1.0 + 0.01 * e).astype(np.float32)
    if w.expert == "mod8":
        return (1.0 + 0.01 * np.mod(e, 8.0)).astype(np.float32)
    raise ValueError(f"unknown expert recipe {w.expert!r}")


def make_inputs(w: Workload, seed: Optional[int] = None,
                with_x: bool = True) -> dict:
    """Draw the seeded inputs of workload ``w``.

    Returns a dict with ``logits`` (fp32 [T,E]), ``x`` (fp32 [T,H] or uint16
    bf16 bits [T,H]; absent when ``with_x`` is False), ``expert_scale`` (fp32
    [E] or None) and, for clustered logits, ``cluster`` (int64 [T]).
    """
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    T, H, E = w.T, w.H, w.E
    noise = rng.standard_normal((T, E), dtype=np.float32)
    out: dict = {}
    if with_x:
        x = rng.standard_normal((T, H), dtype=np.float32)
        out["x"] = x if w.x_dtype == F32 else f32_to_bf16_bits(x)
        del x
    else:
        # keep the draw order identical whether or not x is materialised
        _skip_normals(rng, T * H)
    if w.logits == "normal":
        logits = noise
    elif w.logits == "zipf":
        # expert e has Zipf rank e+1: probability proportional to (e+1)^-s;
        # the normaliser is a constant shift and is dropped.
        bias = (-w.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64)))
        logits = noise + bias.astype(np.float32)[None, :]
    elif w.logits == "clusters":
        per = E // w.n_clusters
        cluster = rng.integers(0, w.n_clusters, size=T)
        member = (np.arange(E)[None, :] // per) == cluster[:, None]
        logits = noise + np.float32(w.cluster_bias) * member.astype(np.float32)
        out["cluster"] = cluster
    else:
        raise ValueError(f"unknown logit recipe {w.logits!r}")
    out["logits"] = np.ascontiguousarray(logits, dtype=np.float32)
    out["expert_scale"] = expert_scale(w)
    return out


def _skip_normals(rng: np.random.Generator, n: int) -> None:
    chunk = 1 << 24
    while n > 0:
        m = min(n, chunk)
        rng.standard_normal(m, dtype=np.float32)
        n -= m


# --------------------------------------------------------------------------
# Adversarial and edge-case logits.  Each returns fp32 [T, E].
# --------------------------------------------------------------------------

def logits_all_equal(T: int, E: int, value: float = 0.25) -> np.ndarray:
    """Every logit equal: every expert ties with every other."""
    return np.full((T, E), value, dtype=np.float32)


def logits_signed_zeros(T: int, E: int, seed: int = 0) -> np.ndarray:
    """Only +0.0, -0.0 and a few +-1.0: ties between the two zeros."""
    rng = np.random.Generator(np.random.PCG64(seed))
    choice = rng.integers(0, 4, size=(T, E))
    table = np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32)
    return table[choice]


def logits_few_levels(T: int, E: int, levels: int = 3,
                      seed: int = 0) -> np.ndarray:
    """Logits drawn from a handful of integer levels: dense ties."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, levels, size=(T, E)).astype(np.float32)


def logits_one_hot_experts(T: int, E: int, K: int, first: int = 0,
                           seed: int = 0) -> np.ndarray:
    """Every token prefers the same K experts (a single hot set)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lg = rng.standard_normal((T, E), dtype=np.float32)
    hot = (np.arange(K) + first) % E
    lg[:, hot] += np.float32(100.0)
    return lg


def logits_masked(T: int, E: int, seed: int = 0) -> np.ndarray:
    """N(0, 1) logits with a share of each token's experts masked to -inf
    (0, 50, 90 or 95 %, drawn per token), then one random expert of every
    token set finite again, so each token keeps at least one finite logit
    and may have fewer than K (its remaining picks are -inf ties)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lg = rng.standard_normal((T, E), dtype=np.float32)
    share = rng.choice(np.array([0.0, 0.5, 0.9, 0.95]), size=T)
    lg[rng.random((T, E)) < share[:, None]] = -np.inf
    lg[np.arange(T), rng.integers(0, E, size=T)] = rng.standard_normal(
        T, dtype=np.float32)
    return lg


def logits_floored(T: int, E: int, G: int, K: int, per_lane: int,
                   seed: int = 0) -> np.ndarray:
    """Logits that put a chosen number of candidates above a lane-maximum
    threshold.  Lanes are the G residues of the expert index mod G, in rows
    of 16; in each row kk = ceil(K / (G/16)) lanes are high: one holds a
    single logit just above 10 (so it is the row's kk-th largest lane
    maximum), each other holds `per_lane` logits in [10.5, 11); every other
    logit is N(0, 1).  So (G/16) * (1 + (kk - 1) * per_lane) logits reach the
    smallest such maximum.  Values are distinct with probability one (no
    ties).  E must be a multiple of G."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lg = rng.standard_normal((T, E), dtype=np.float32)
    C = E // G
    rows = G // 16
    kk = -(-K // rows)
    for t in range(T):
        for r in range(rows):
            lanes = r * 16 + rng.choice(16, kk, replace=False)
            j = int(rng.integers(C))
            lg[t, lanes[0] + G * j] = np.float32(10.0 + rng.random() * 1e-3)
            for sub in lanes[1:]:
                js = rng.choice(C, per_lane, replace=False)
                lg[t, sub + G * js] = (10.5 + 0.5 * rng.random(per_lane)
                                       ).astype(np.float32)
    return lg


def random_x(T: int, H: int, dtype: str, seed: int = 0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((T, H), dtype=np.float32)
    return x if dtype == F32 else f32_to_bf16_bits(x)


def random_topk_idx(T: int, E: int, K: int, seed: int = 0) -> np.ndarray:
    """K distinct expert ids per token, uniformly at random (int32 [T,K])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1)[:, :K].astype(np.int32)


def replica_layout(E: int, G: int, rho: float, seed: int = 0) -> np.ndarray:
    """A seeded expert layout with replicas: holds[r, e] = 1 when rank r has a
    replica of expert e (uint8 [G, E]).

    Every expert keeps its contiguous home rank e // (E/G); then round(rho*E)
    extra replicas go, one at a time, to a uniformly drawn expert and a
    uniformly drawn rank that does not hold it yet and has a free slot, with
    at most ceil((1 + rho) * E / G) replicas per rank (the replica budget of
    "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
    Training", Section 3.1).  Stands in for the planner's layout, which is
    not built.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    holds = np.zeros((G, E), np.uint8)
    holds[np.arange(E) // (E // G), np.arange(E)] = 1
    budget = int(np.ceil((1.0 + rho) * E / G))
    extra = int(round(rho * E))
    placed = 0
    tries = 0
    while placed < extra and tries < 100 * max(extra, 1):
        tries += 1
        e = int(rng.integers(0, E))
        free = np.nonzero((holds[:, e] == 0) & (holds.sum(axis=1) < budget))[0]
        if len(free) == 0:
            continue
        holds[int(rng.choice(free)), e] = 1
        placed += 1
    return holds


def assign_draws(T: int, K: int, seed: int = 0):
    """Uniform uint32 draws for the task assignment's random choices:
    (u_node, u_rank), each uint32 [T, K]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.integers(0, 1 << 32, size=(2, T, K), dtype=np.uint64)
    return u[0].astype(np.uint32), u[1].astype(np.uint32)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [
    "Workload", "WORKLOADS", "TINY", "MIXTRAL", "QWEN3", "DEEPSEEK_V3",
    "DEEPSEEK_V3_DECODE", "KIMI", "F32", "BF16", "make_inputs",
    "expert_scale", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "logits_all_equal", "logits_signed_zeros", "logits_few_levels",
    "logits_one_hot_experts", "random_x", "random_topk_idx", "ceil_div",
    "replica_layout", "assign_draws",
]
