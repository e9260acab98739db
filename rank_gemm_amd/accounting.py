"""Algorithmic FLOP and byte counts of the mixed-adapter LoRA linear.

These are the figures the benchmark divides by kernel time. They count what
the method must compute and move, at each adapter's true rank:

* base GEMM: 2*T*d_in*d_out FLOP; bytes es*(T*d_in + d_in*d_out + T*d_out).
* correction: sum over adapter rows of 2*r_s*(d_in + d_out) FLOP.
* shrink + expand bytes: the adapter rows of x, each active slot's A_s and
  B_s once at true rank, the fp32 intermediate written and read once
  (T_a * r_max * 4 * 2) and the read-modify-write of the adapter rows of y.

Closed forms of "LoRA serving, embeddings, rerankers, pooling"
(mlinterviewnotes.com), sections "Adapter size" and the paragraph on the
rank-16 correction's share of a square projection, are reproduced by the
functions below and checked in the CPU tests.
"""
from __future__ import annotations

import numpy as np

# Llama-3-8B projection shapes (d_in, d_out): d = 4096, d_kv = 1024,
# FFN 14336, 32 layers (symbol list of the mlinterviewnotes page).
LLAMA3_8B_LAYERS = 32
LLAMA3_8B_TARGETS = {
    "q_proj": (4096, 4096),
    "k_proj": (4096, 1024),
    "v_proj": (4096, 1024),
    "o_proj": (4096, 4096),
    "gate_proj": (4096, 14336),
    "up_proj": (4096, 14336),
    "down_proj": (14336, 4096),
}
ATTENTION_TARGETS = ("q_proj", "k_proj", "v_proj", "o_proj")

ES = {"bf16": 2, "f32": 4}


def adapter_params(r: int, d_in: int, d_out: int) -> int:
    """Parameters of one adapter on one linear: r*(d_in + d_out)."""
    return r * (d_in + d_out)


def layer_width_sum(targets=None) -> int:
    """Sum of (d_in + d_out) over a decoder layer's adapted targets."""
    names = targets or LLAMA3_8B_TARGETS.keys()
    return sum(sum(LLAMA3_8B_TARGETS[n]) for n in names)


def model_adapter_params(r: int, targets=None, layers: int = LLAMA3_8B_LAYERS) -> int:
    return r * layers * layer_width_sum(targets)


def model_adapter_bytes(r: int, targets=None, layers: int = LLAMA3_8B_LAYERS, es: int = 2) -> int:
    return es * model_adapter_params(r, targets, layers)


def base_flops(T: int, d_in: int, d_out: int) -> int:
    return 2 * T * d_in * d_out


def correction_flops_per_row(r: int, d_in: int, d_out: int) -> int:
    return 2 * r * (d_in + d_out)


def correction_to_base_ratio(r: int, d_in: int, d_out: int) -> float:
    """FLOP share of the rank-r correction for one row of a d_in -> d_out linear."""
    return correction_flops_per_row(r, d_in, d_out) / (2 * d_in * d_out)


def base_bytes(T: int, d_in: int, d_out: int, es: int) -> int:
    return es * (T * d_in + d_in * d_out + T * d_out)


def segments(slot_ids, ranks):
    """{slot: row count} for slots >= 1 whose rank is > 0."""
    slot_ids = np.asarray(slot_ids)
    ranks = np.asarray(ranks)
    out = {}
    for s, n in zip(*np.unique(slot_ids, return_counts=True)):
        if s != 0 and ranks[s] > 0:
            out[int(s)] = int(n)
    return out


def correction_flops(slot_ids, ranks, d_in: int, d_out: int) -> int:
    return sum(n * correction_flops_per_row(int(ranks[s]), d_in, d_out) for s, n in segments(slot_ids, ranks).items())


def correction_bytes(slot_ids, ranks, d_in: int, d_out: int, es: int, r_max: int, padded: bool = False) -> int:
    """Shrink + expand algorithmic bytes (see module docstring). ``padded``
    counts A and B at r_max instead of the true rank."""
    seg = segments(slot_ids, ranks)
    T_a = sum(seg.values())
    w = sum(es * (r_max if padded else int(ranks[s])) * (d_in + d_out) for s in seg)
    return es * T_a * d_in + w + 2 * 4 * T_a * r_max + 2 * es * T_a * d_out


def call_flops(slot_ids, ranks, d_in, d_out) -> int:
    return base_flops(len(slot_ids), d_in, d_out) + correction_flops(slot_ids, ranks, d_in, d_out)


def call_bytes(slot_ids, ranks, d_in, d_out, es, r_max) -> int:
    """Base GEMM bytes plus shrink/expand bytes of one lora_linear call."""
    return base_bytes(len(slot_ids), d_in, d_out, es) + correction_bytes(slot_ids, ranks, d_in, d_out, es, r_max)
