"""GPU parity of the correction alone (lora_delta over plans of every chunk
size, lora_delta_bgmv token by token) against the fp64 oracle.

Two checks per case:
* from y = 0, the call leaves bf16(delta) in adapter rows: compared element
  by element with the oracle's y - x W^T within one bf16 ulp of the delta
  plus fp32 accumulation error; rows on slot 0, on a rank-0 slot or with an
  id outside [1, S) stay exactly zero;
* from y = the bf16 base output of lora_linear with a base-only plan, the
  call gives the layer: compared with the oracle's y by the graded bound and
  the per-element rounding bound (base rounded, then base + delta rounded).
"""
import numpy as np
import pytest
import torch

from rank_gemm_amd import lora
from rank_gemm_amd.inputs import make_config, make_custom

from gpu_util import bf16_ulp, build_pool, check_close, oracle_pair, to_f64

pytestmark = pytest.mark.gpu

CHUNKS = (16, 32, 64, 128)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    lora.lib()
    yield


def _cases():
    g = np.random.default_rng(5)
    long_ids = np.repeat(g.integers(0, 5, size=8), 125).astype(np.int32)  # long segments, a base block
    return {
        "decode q_proj": lambda: make_config(2),
        "k/v mixed ranks": lambda: make_config(4),
        "o_proj 50 adapters": lambda: make_config(5),
        "long segments": lambda: make_custom(41, 1000, 1024, 520, 5, [0, 16, 8, 16, 4], [0, 32, 16, 32, 8],
                                             long_ids),
        "ranks past 64": lambda: make_custom(42, 300, 264, 200, 4, [0, 80, 17, 0], [0, 160, 34, 0],
                                             g.integers(0, 4, size=300).astype(np.int32), r_max=80),
    }


CASES = _cases()


def _delta_check(w, proj, y, ids, label):
    ref, base = oracle_pair(w, proj, slot_ids=ids)
    d_ref = ref - base
    yh = to_f64(y)
    ranks = w.ranks
    adapted = np.array([0 < s < w.S and ranks[s] > 0 for s in ids])
    assert np.all(yh[~adapted] == 0), f"{label}: rows without an adapter were touched"
    scale = np.max(np.abs(d_ref)) if d_ref.size else 0.0
    bound = bf16_ulp(np.abs(d_ref)) + 1e-5 * scale
    bad = np.abs(yh - d_ref) > bound
    err = float(np.max(np.abs(yh - d_ref)) / (scale if scale > 0 else 1.0))
    print(f"[delta] {label}: rel err of the delta {err:.3e}", flush=True)
    assert not bad.any(), f"{label}: {int(bad.sum())} delta elements outside one bf16 ulp"
    return ref, base


def _base_output(w, proj, pool, x, W):
    pb = lora.plan(np.zeros(w.T, np.int32), w.S)
    return lora.linear(x, W, pool, pb)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("chunk", CHUNKS)
def test_delta_sgmv_chunks(name, chunk):
    w = CASES[name]()
    proj = w.projections[0]
    pool = build_pool(w, proj)
    x = lora.to_device(proj.x, "bf16")
    W = lora.to_device(proj.W, "bf16")
    p = lora.plan(w.slot_ids, w.S, chunk=chunk)
    assert p.info.chunk == chunk
    y = torch.zeros((w.T, proj.d_out), dtype=torch.bfloat16, device="cuda")
    lora.correction(x, pool, p, y)
    torch.cuda.synchronize()
    ref, base = _delta_check(w, proj, y, w.slot_ids, f"{name} chunk {chunk}")
    y = _base_output(w, proj, pool, x, W)
    lora.correction(x, pool, p, y)
    torch.cuda.synchronize()
    check_close(to_f64(y), ref, "bf16", f"{name} chunk {chunk}: base + delta", base)


@pytest.mark.parametrize("name", list(CASES))
def test_delta_bgmv(name):
    w = CASES[name]()
    proj = w.projections[0]
    pool = build_pool(w, proj)
    x = lora.to_device(proj.x, "bf16")
    W = lora.to_device(proj.W, "bf16")
    ids_dev = torch.from_numpy(w.slot_ids.copy()).cuda()
    y = torch.zeros((w.T, proj.d_out), dtype=torch.bfloat16, device="cuda")
    lora.correction_bgmv(x, pool, ids_dev, y)
    torch.cuda.synchronize()
    ref, base = _delta_check(w, proj, y, w.slot_ids, f"{name} bgmv")
    y = _base_output(w, proj, pool, x, W)
    lora.correction_bgmv(x, pool, ids_dev, y)
    torch.cuda.synchronize()
    check_close(to_f64(y), ref, "bf16", f"{name} bgmv: base + delta", base)


def test_delta_bgmv_ids_out_of_range():
    """Ids outside [1, S) (and slot 0) leave their rows of y unchanged."""
    w = make_custom(43, 64, 256, 96, 4, [0, 8, 4, 8], [0, 16, 8, 16],
                    np.random.default_rng(3).integers(0, 4, size=64).astype(np.int32), r_max=8)
    proj = w.projections[0]
    pool = build_pool(w, proj)
    ids = w.slot_ids.copy()
    ids[::7] = -1
    ids[3::11] = 4
    ids[5::13] = 1 << 20
    x = lora.to_device(proj.x, "bf16")
    y = torch.zeros((w.T, proj.d_out), dtype=torch.bfloat16, device="cuda")
    lora.correction_bgmv(x, pool, torch.from_numpy(ids).cuda(), y)
    torch.cuda.synchronize()
    kept = np.where((ids >= 1) & (ids < 4), ids, 0).astype(np.int32)
    _delta_check(w, proj, y, kept, "bgmv ids out of range")


@pytest.mark.parametrize("dtype,d_in", [("f32", 256), ("bf16", 515)])
@pytest.mark.parametrize("chunk", [16, 64])
def test_delta_element_generic(dtype, d_in, chunk):
    """fp32 pools and bf16 pools with d_in % 8 != 0 take the element-generic
    shrink and expand (items of any row count)."""
    T, S, ranks = 150, 5, [0, 8, 5, 0, 8]
    ids = np.repeat(np.random.default_rng(6).integers(0, S, size=6), 25).astype(np.int32)
    w = make_custom(44, T, d_in, 130, S, ranks, [2.0 * r for r in ranks], ids, dtype=dtype, r_max=8)
    proj = w.projections[0]
    pool = build_pool(w, proj)
    x = lora.to_device(proj.x, dtype)
    W = lora.to_device(proj.W, dtype)
    p = lora.plan(ids, S, chunk=chunk)
    y = _base_output(w, proj, pool, x, W)
    lora.correction(x, pool, p, y)
    torch.cuda.synchronize()
    ref, base = oracle_pair(w, proj)
    check_close(to_f64(y), ref, dtype, f"generic {dtype} d_in={d_in} chunk {chunk}",
                base if dtype == "bf16" else None)
    if dtype == "bf16":
        with pytest.raises(lora.LoraError):
            lora.correction_bgmv(x, pool, torch.from_numpy(ids).cuda(), y)


def test_linear_refuses_chunked_plan():
    w = make_config(2)
    proj = w.projections[0]
    pool = build_pool(w, proj)
    p = lora.plan(w.slot_ids, w.S, chunk=64)
    with pytest.raises(lora.LoraError) as e:
        lora.linear(lora.to_device(proj.x, "bf16"), lora.to_device(proj.W, "bf16"), pool, p)
    assert e.value.status == lora.LORA_EINVAL
