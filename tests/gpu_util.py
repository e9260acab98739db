"""Helpers of the GPU parity tests: drive liblora through its binding and
compare with the fp64 oracle on the same seeded host inputs."""
import numpy as np
import torch

import oracle
from rank_gemm_amd import lora
from rank_gemm_amd.inputs import bf16_to_f32

TOL = {"f32": 1e-5, "bf16": 2e-2}  # max|y - y_ref| / max|y_ref|


def build_pool(w, proj, device="cuda"):
    pool = lora.Pool(w.S, w.r_max, proj.d_in, proj.d_out, w.dtype, device)
    for s, a in sorted(proj.adapters.items()):
        pool.install(s, lora.to_device(a.A, w.dtype, device), lora.to_device(a.B, w.dtype, device), a.alpha)
    return pool


def run_layer(w, proj, pool=None, slot_ids=None, y=None, device="cuda"):
    """One lora_linear call on the device; returns (y tensor, pool, plan)."""
    pool = pool or build_pool(w, proj, device)
    ids = w.slot_ids if slot_ids is None else slot_ids
    p = lora.plan(ids, w.S, device)
    x = lora.to_device(proj.x, w.dtype, device)
    W = lora.to_device(proj.W, w.dtype, device)
    y = lora.linear(x, W, pool, p, y=y)
    torch.cuda.synchronize()
    return y, pool, p


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_rows(w, proj, rows=None, slot_ids=None, want_h=False):
    ids = w.slot_ids if slot_ids is None else slot_ids
    return oracle.lora_rows(w.dtype, proj.x, proj.W, w.S, proj.adapters, ids, rows=rows, want_h=want_h,
                            h_width=w.r_max)


def oracle_pair(w, proj, rows=None, slot_ids=None):
    """(y_ref, base_ref): the oracle's output and its base-only output x W^T,
    both from one pass of the oracle over W."""
    ids = w.slot_ids if slot_ids is None else slot_ids
    return oracle.lora_rows(w.dtype, proj.x, proj.W, w.S, proj.adapters, ids, rows=rows, want_base=True)


def rel_err(y, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0))


def bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_close(y, ref, dtype, label="", base_ref=None):
    """The graded bound, plus (bf16, when the oracle's base output base_ref is
    given) a per-element bound that follows from the arithmetic: y is the
    base rounded to bf16, plus the fp32 correction, rounded again, so each
    element is within half an ulp at |base| plus half an ulp at |y|, i.e. one
    ulp at the larger of the two, plus fp32 accumulation error."""
    err = rel_err(y, ref)
    print(f"[parity] {label} dtype={dtype} rel_err={err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert err <= TOL[dtype], f"{label}: rel err {err:.3e} > {TOL[dtype]}"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if dtype == "bf16":
        if base_ref is None:
            return err
        big = np.maximum(np.abs(ref), np.abs(base_ref))
        bound = bf16_ulp(big) + 1e-4 * scale
    else:
        bound = TOL["f32"] * scale
    bad = np.abs(y - ref) > bound
    assert not bad.any(), f"{label}: {int(bad.sum())} elements outside the rounding bound"
    return err


def sample_rows(slot_ids, n, seed=0):
    """Rows for the oracle at full size: the first and last row of every
    segment plus seeded random rows."""
    g = np.random.default_rng(seed)
    T = len(slot_ids)
    order = np.argsort(slot_ids, kind="stable")
    bounds = np.flatnonzero(np.diff(slot_ids[order])) + 1
    ends = set([int(order[0]), int(order[-1])])
    for b in bounds:
        ends.add(int(order[b - 1]))
        ends.add(int(order[b]))
    rows = sorted(ends | set(g.choice(T, size=min(n, T), replace=False).tolist()))
    return np.array(rows, np.int32)


def host_values(arr, dtype):
    return bf16_to_f32(arr).astype(np.float64) if dtype == "bf16" else np.asarray(arr, np.float64)
