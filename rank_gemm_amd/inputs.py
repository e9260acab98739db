"""Seeded synthetic workloads for the mixed-adapter LoRA linear.

This module draws inputs only: token-to-slot maps, activations, base weights
and adapter factors, as host numpy arrays. It holds none of the layer's
arithmetic, so that the GPU path and the CPU oracle can both be fed from it
without sharing any computation.

Shapes follow the Llama-3-8B dimensions of "LoRA serving, embeddings,
rerankers, pooling" (mlinterviewnotes.com), section "LoRA serving ...",
symbol list: d = 4096, d_kv = 1024, FFN intermediate 14336.

Every array has its own generator, ``numpy.random.default_rng([seed, proj,
tag])`` (PCG64), so arrays are independent of draw order and can be drawn on
several threads. Distributions:

* x ~ N(0, 1), W ~ N(0, 0.02), B_s ~ N(0, 0.02) (0.02 is the standard
  deviation), A_s ~ U[-1/sqrt(d_in), 1/sqrt(d_in)); all drawn in float32.
* bf16 arrays are the float32 draws rounded to nearest, ties to even, and
  are handed out as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32 = "f32"
BF16 = "bf16"

# tags of the per-array generators
_TAG_SLOTS, _TAG_X, _TAG_W = 0, 1, 2


def _tag_a(s: int) -> int:
    return 3 + 2 * s


def _tag_b(s: int) -> int:
    return 4 + 2 * s


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.

    Inputs are finite draws, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    t = (u >> np.uint32(16)) & np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Adapter:
    rank: int
    alpha: float
    A: np.ndarray  # [rank, d_in], dtype float32 or uint16 (bf16 bits)
    B: np.ndarray  # [d_out, rank]


@dataclasses.dataclass
class Projection:
    name: str
    d_in: int
    d_out: int
    x: np.ndarray  # [T, d_in]
    W: np.ndarray  # [d_out, d_in]
    adapters: dict  # slot -> Adapter, slots 1..S-1 that are installed


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    T: int
    S: int
    r_max: int
    slot_ids: np.ndarray  # int32 [T]
    projections: list

    @property
    def ranks(self) -> np.ndarray:
        """int32 [S]: the installed rank of every slot, 0 for slot 0."""
        r = np.zeros(self.S, np.int32)
        for s, a in self.projections[0].adapters.items():
            r[s] = a.rank
        return r


def _normal(seed, shape, std):
    g = np.random.default_rng(seed)
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _uniform(seed, shape, lo, hi):
    g = np.random.default_rng(seed)
    a = g.random(shape, dtype=np.float32)
    a *= np.float32(hi - lo)
    a += np.float32(lo)
    return a


def _cast(a, dtype):
    return bf16_bits(a) if dtype == BF16 else a


def _projection(seed, pidx, name, T, d_in, d_out, dtype, ranks, alphas, x=None, pool=None):
    """Draw one projection: its input (unless shared), base weight and adapters."""
    jobs = {}
    pool = pool or ThreadPoolExecutor(8)
    if x is None:
        jobs["x"] = pool.submit(lambda: _cast(_normal([seed, pidx, _TAG_X], (T, d_in), 1.0), dtype))
    jobs["W"] = pool.submit(lambda: _cast(_normal([seed, pidx, _TAG_W], (d_out, d_in), 0.02), dtype))
    bound = 1.0 / np.sqrt(d_in)

    def adapter(s):
        r = int(ranks[s])
        A = _cast(_uniform([seed, pidx, _tag_a(s)], (r, d_in), -bound, bound), dtype)
        B = _cast(_normal([seed, pidx, _tag_b(s)], (d_out, r), 0.02), dtype)
        return Adapter(r, float(alphas[s]), A, B)

    ad = {s: pool.submit(adapter, s) for s in range(1, len(ranks)) if ranks[s] > 0}
    xv = jobs["x"].result() if x is None else x
    return Projection(name, d_in, d_out, xv, jobs["W"].result(), {s: f.result() for s, f in ad.items()})


def _zipf_slots(g, n, n_slots, a):
    p = np.arange(1, n_slots + 1, dtype=np.float64) ** (-a)
    p /= p.sum()
    return g.choice(np.arange(1, n_slots + 1), size=n, p=p)


# Config table. "alpha" is per slot; slot 0 is the zero adapter (rank 0).
CONFIG_NAMES = {
    1: "tiny fp32: T=64, 256->256, S=5 (rank 8, alpha 16), uniform slots",
    2: "llama3-8b q_proj decode bf16: T=64, 4096->4096, S=9 (rank 16, alpha 32), 8 adapters x 8 tokens shuffled",
    3: "llama3-8b gate/up prefill bf16: T=8192 (16 seqs x 512), 4096->14336 x2, S=17 (rank 16, alpha 32)",
    4: "llama3-8b k/v mixed ranks bf16: T=256, 4096->1024 x2 (k_proj, v_proj on one x), S=33 (ranks {8,16,32,64}, "
       "r_max 64, alpha 2r), Zipf(1.1), 20% base rows",
    5: "llama3-8b o_proj + down_proj bf16: T=512, 4096->4096 and 14336->4096, S=129 (rank 16, alpha 32), 50 active adapters",
}


def make_config(i: int, seed: int | None = None, layer: int = 0, pool=None) -> Workload:
    """Draw workload ``i`` (1..5). ``seed`` defaults to ``i``; ``layer`` picks an
    independent set of weights with the same slot structure (used to model
    the layers of one decode step)."""
    seed = i if seed is None else seed
    own_pool = pool is None
    pool = pool or ThreadPoolExecutor(8)
    try:
        g = np.random.default_rng([seed, _TAG_SLOTS])
        # every layer shares the slot structure, weights differ per layer
        wseed = seed if layer == 0 else seed * 1000003 + layer
        if i == 1:
            T, S, r, dt = 64, 5, 8, F32
            ranks = np.array([0] + [r] * (S - 1), np.int32)
            alphas = np.array([0.0] + [16.0] * (S - 1))
            slot_ids = g.integers(0, S, size=T).astype(np.int32)
            projs = [_projection(wseed, 0, "proj", T, 256, 256, dt, ranks, alphas, pool=pool)]
            return Workload(CONFIG_NAMES[1], dt, T, S, r, slot_ids, projs)
        if i == 2:
            T, S, r, dt = 64, 9, 16, BF16
            ranks = np.array([0] + [r] * (S - 1), np.int32)
            alphas = np.array([0.0] + [32.0] * (S - 1))
            slot_ids = g.permutation(np.repeat(np.arange(1, 9), 8)).astype(np.int32)
            projs = [_projection(wseed, 0, "q_proj", T, 4096, 4096, dt, ranks, alphas, pool=pool)]
            return Workload(CONFIG_NAMES[2], dt, T, S, r, slot_ids, projs)
        if i == 3:
            T, S, r, dt = 8192, 17, 16, BF16
            ranks = np.array([0] + [r] * (S - 1), np.int32)
            alphas = np.array([0.0] + [32.0] * (S - 1))
            seq_slots = g.integers(0, S, size=16)
            slot_ids = np.repeat(seq_slots, 512).astype(np.int32)
            gate = _projection(wseed, 0, "gate_proj", T, 4096, 14336, dt, ranks, alphas, pool=pool)
            up = _projection(wseed, 1, "up_proj", T, 4096, 14336, dt, ranks, alphas, x=gate.x, pool=pool)
            return Workload(CONFIG_NAMES[3], dt, T, S, r, slot_ids, [gate, up])
        if i == 4:
            T, S, r_max, dt = 256, 33, 64, BF16
            ranks = np.concatenate([[0], g.choice([8, 16, 32, 64], size=S - 1)]).astype(np.int32)
            alphas = 2.0 * ranks
            slot_ids = np.zeros(T, np.int32)
            n_base = int(round(0.2 * T))
            base_pos = g.choice(T, size=n_base, replace=False)
            rest = np.setdiff1d(np.arange(T), base_pos)
            slot_ids[rest] = _zipf_slots(g, len(rest), S - 1, 1.1)
            k = _projection(wseed, 0, "k_proj", T, 4096, 1024, dt, ranks, alphas, pool=pool)
            v = _projection(wseed, 1, "v_proj", T, 4096, 1024, dt, ranks, alphas, x=k.x, pool=pool)
            return Workload(CONFIG_NAMES[4], dt, T, S, r_max, slot_ids, [k, v])
        if i == 5:
            T, S, r, dt = 512, 129, 16, BF16
            ranks = np.array([0] + [r] * (S - 1), np.int32)
            alphas = np.array([0.0] + [32.0] * (S - 1))
            active = g.choice(np.arange(1, S), size=50, replace=False)
            slot_ids = g.choice(active, size=T).astype(np.int32)
            o = _projection(wseed, 0, "o_proj", T, 4096, 4096, dt, ranks, alphas, pool=pool)
            down = _projection(wseed, 1, "down_proj", T, 14336, 4096, dt, ranks, alphas, pool=pool)
            return Workload(CONFIG_NAMES[5], dt, T, S, r, slot_ids, [o, down])
        raise ValueError(f"unknown config {i}")
    finally:
        if own_pool:
            pool.shutdown()


def make_custom(seed, T, d_in, d_out, S, ranks, alphas, slot_ids, dtype=BF16, r_max=None, pool=None) -> Workload:
    """A workload of arbitrary shape for edge-case tests (ragged T, odd widths,
    empty segments, rank-0 slots). ``ranks[s] == 0`` leaves slot s empty."""
    ranks = np.asarray(ranks, np.int32)
    slot_ids = np.asarray(slot_ids, np.int32)
    own_pool = pool is None
    pool = pool or ThreadPoolExecutor(8)
    try:
        p = _projection(seed, 0, "proj", T, d_in, d_out, dtype, ranks, np.asarray(alphas, np.float64), pool=pool)
    finally:
        if own_pool:
            pool.shutdown()
    rm = int(r_max if r_max is not None else max(1, int(ranks.max(initial=0))))
    return Workload("custom", dtype, T, S, rm, slot_ids, [p])


def make_slices(seed, T, d_in, d_outs, S, ranks, alphas, slot_ids, dtype=BF16, r_max=None, names=None,
                pool=None) -> Workload:
    """Several projections that read one x (a merged q/k/v or gate/up): one
    projection per entry of ``d_outs``, each with its own base weight and its
    own adapters. ``ranks`` and ``alphas`` are [n][S] (per-slice ranks of the
    same slot may differ; 0 leaves the slot empty in that slice)."""
    slot_ids = np.asarray(slot_ids, np.int32)
    ranks = [np.asarray(r, np.int32) for r in ranks]
    names = names or [f"slice{i}" for i in range(len(d_outs))]
    own_pool = pool is None
    pool = pool or ThreadPoolExecutor(8)
    try:
        first = _projection(seed, 0, names[0], T, d_in, d_outs[0], dtype, ranks[0], np.asarray(alphas[0], np.float64),
                            pool=pool)
        projs = [first]
        for i in range(1, len(d_outs)):
            projs.append(_projection(seed, i, names[i], T, d_in, d_outs[i], dtype, ranks[i],
                                     np.asarray(alphas[i], np.float64), x=first.x, pool=pool))
    finally:
        if own_pool:
            pool.shutdown()
    rm = int(r_max if r_max is not None else max(1, max(int(r.max(initial=0)) for r in ranks)))
    return Workload("slices", dtype, T, S, rm, slot_ids, projs)


def make_qkv_decode(seed: int = 2, layer: int = 0, pool=None) -> Workload:
    """The q/k/v projections of one Llama-3-8B attention layer at decode: the
    slot structure of the q_proj decode workload (T=64, S=9, rank 16, alpha
    32, 8 adapters x 8 tokens shuffled) with k and v of width d_kv = 1024."""
    g = np.random.default_rng([seed, _TAG_SLOTS])
    T, S, r = 64, 9, 16
    slot_ids = g.permutation(np.repeat(np.arange(1, 9), 8)).astype(np.int32)
    ranks = np.array([0] + [r] * (S - 1), np.int32)
    alphas = np.array([0.0] + [32.0] * (S - 1))
    wseed = seed if layer == 0 else seed * 1000003 + layer
    return make_slices(wseed * 101 + 7, T, 4096, [4096, 1024, 1024], S, [ranks] * 3, [alphas] * 3, slot_ids,
                       names=["q_proj", "k_proj", "v_proj"], pool=pool)
