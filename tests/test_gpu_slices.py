"""GPU parity of lora_linear_multi: several projections that read one x (a
merged q/k/v or gate/up), each with its own base weight, output and pool,
against the fp64 oracle applied to each projection on its own.

The bar is that of lora_linear (relative error and per-element rounding
bound). Where the concatenated columns take the decode path, the slices
must share one GEMM launch and one epilogue launch; that is checked with
the library's per-kernel profiler.
"""
import ctypes

import numpy as np
import pytest
import torch

from rank_gemm_amd import lora
from rank_gemm_amd.inputs import make_qkv_decode, make_slices

from gpu_util import build_pool, check_close, oracle_pair, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    lora.lib()
    yield


def run_multi(w, slot_ids=None, profile=False):
    ids = w.slot_ids if slot_ids is None else slot_ids
    pools = [build_pool(w, pr) for pr in w.projections]
    p = lora.plan(ids, w.S)
    x = lora.to_device(w.projections[0].x, w.dtype)
    Ws = [lora.to_device(pr.W, w.dtype) for pr in w.projections]
    ys = [torch.full((w.T, pr.d_out), float("nan"), dtype=x.dtype, device="cuda") for pr in w.projections]
    torch.cuda.synchronize()
    if profile:
        lora.profile_begin()
    ys = lora.linear_multi(x, Ws, pools, p, ys=ys)
    stats = lora.profile_end() if profile else None
    torch.cuda.synchronize()
    return ys, pools, stats


def check_slices(w, ys, label, slot_ids=None):
    for pr, y in zip(w.projections, ys):
        ref, base = oracle_pair(w, pr, slot_ids=slot_ids)
        yh = to_f64(y)
        assert np.isfinite(yh).all(), f"{label} {pr.name}: non-finite output"
        check_close(yh, ref, w.dtype, f"{label} {pr.name}", base if w.dtype == "bf16" else None)


def test_qkv_decode_one_pass():
    """q/k/v of a decode step: one GEMM launch and one epilogue for all three."""
    w = make_qkv_decode()
    ys, _, stats = run_multi(w, profile=True)
    print(f"[slices] qkv kernels: { {k: v['count'] for k, v in stats.items()} }", flush=True)
    assert stats["gemm_splitk"]["count"] == 1
    assert stats["gemm_splitk_epilogue"]["count"] == 1
    check_slices(w, ys, "qkv decode")


@pytest.mark.parametrize("r_max", [16, 12])
def test_ragged_widths_and_per_slice_ranks(r_max):
    """Slice widths that end mid-tile, a K tail, a ragged row tile, ranks that
    differ per slice for the same slot, and a slice with no adapter at all."""
    S = 6
    ranks = [[0, 16, 8, 0, 4, 12], [0, 8, 12, 12, 0, 1], [0, 0, 0, 0, 0, 0]]
    ranks = [[min(r, r_max) for r in rr] for rr in ranks]
    alphas = [[2.0 * r for r in rr] for rr in ranks]
    g = np.random.default_rng(11)
    T = 70
    ids = g.integers(0, S, size=T).astype(np.int32)
    w = make_slices(31 + r_max, T, 1032, [1000, 72, 200], S, ranks, alphas, ids, r_max=r_max)
    ys, _, stats = run_multi(w, profile=True)
    assert stats["gemm_splitk"]["count"] == 1
    check_slices(w, ys, f"ragged r_max={r_max}")


def test_heavy_shrink_slices_mixed_ranks():
    """Many adapters with ranks up to 64 that differ per slice: the shrink
    runs as shrink tiles of one item each (ranks 48 to 64 fill a tile), for
    all three slices in the one GEMM launch."""
    S = 21
    g = np.random.default_rng(23)
    ranks = [[0] + [int(v) for v in g.integers(1, 65, size=S - 1)] for _ in range(3)]
    ranks[1][3] = 0  # a slot with no adapter in one slice only
    alphas = [[2.0 * r for r in rr] for rr in ranks]
    T = 200
    ids = g.integers(0, S, size=T).astype(np.int32)
    w = make_slices(61, T, 2056, [1024, 256, 200], S, ranks, alphas, ids, r_max=64)
    ys, _, stats = run_multi(w, profile=True)
    assert stats["gemm_splitk"]["count"] == 1
    check_slices(w, ys, "heavy shrink slices")


def test_four_slices_and_base_only_plan():
    """The maximum slice count; then a plan with no adapter row."""
    S = 5
    ranks = [[0, 16, 16, 16, 16]] * 4
    alphas = [[0.0, 32.0, 32.0, 32.0, 32.0]] * 4
    ids = np.array([1, 2, 3, 4, 0, 0, 2, 2, 1, 3, 4, 4, 0, 1, 2, 3], np.int32)
    w = make_slices(45, 16, 2048, [512, 576, 512, 96], S, ranks, alphas, ids, r_max=16)
    ys, pools, stats = run_multi(w, profile=True)
    assert stats["gemm_splitk"]["count"] == 1
    check_slices(w, ys, "four slices")
    zeros = np.zeros_like(ids)
    ys0, _, _ = run_multi(w, slot_ids=zeros)
    check_slices(w, ys0, "four slices, base only", slot_ids=zeros)


def test_prefill_sized_slices_run_one_by_one():
    """Slices whose concatenated columns take the tiled path run separately."""
    S = 9
    ranks = [[0] + [16] * 8] * 2
    alphas = [[0.0] + [32.0] * 8] * 2
    g = np.random.default_rng(3)
    T = 1024
    ids = np.repeat(g.integers(0, S, size=8), 128).astype(np.int32)
    w = make_slices(52, T, 512, [2048, 2048], S, ranks, alphas, ids, r_max=16)
    ys, _, stats = run_multi(w, profile=True)
    assert "gemm_splitk" not in stats
    assert stats["gemm_bf16"]["count"] == 2
    check_slices(w, ys, "prefill slices")


@pytest.mark.parametrize("r_max,n_slices", [(16, 2), (32, 3)])
def test_prefill_slices_share_one_shrink(r_max, n_slices):
    """Slices that all take the tiled path, with enough work items, share one
    shrink launch (x rows read once for every slice's A); each slice's output
    equals, bit for bit, that of its own lora_linear call. Per-slice ranks
    differ for the same slot (one slot is empty in one slice only, ranks not
    multiples of 16), so a group of four rank blocks mixes slices."""
    S = 9
    g = np.random.default_rng(40 + r_max)
    ranks = [[0] + [r_max] * 8]
    ranks.append([0, 8, r_max, 0, 4, r_max, 12, r_max, 8])
    ranks.append([0, 5, 16, r_max, 0, 24, r_max, 1, r_max])
    ranks = [[min(r, r_max) for r in rr] for rr in ranks[:n_slices]]
    alphas = [[2.0 * r for r in rr] for rr in ranks]
    T = 4096
    ids = np.repeat(g.integers(0, S, size=T // 256), 256).astype(np.int32)
    d_outs = [2048, 1536, 1000][:n_slices]
    w = make_slices(70 + r_max, T, 520, d_outs, S, ranks, alphas, ids, r_max=r_max)
    ys, pools, stats = run_multi(w, profile=True)
    assert stats["sgmv_shrink"]["count"] == 1 and stats["gemm_bf16"]["count"] == n_slices, stats
    p = lora.plan(ids, S)
    x = lora.to_device(w.projections[0].x, w.dtype)
    for i, pr in enumerate(w.projections):
        W = lora.to_device(pr.W, w.dtype)
        y1 = lora.linear(x, W, pools[i], p)
        torch.cuda.synchronize()
        assert torch.equal(y1, ys[i]), f"slice {i}: one shared shrink differs from the slice's own call"
    check_slices(w, ys, f"shared shrink r_max={r_max}")


def test_f32_slices():
    S = 5
    ranks = [[0, 8, 8, 8, 8], [0, 8, 0, 4, 8]]
    alphas = [[0.0, 16.0, 16.0, 16.0, 16.0], [0.0, 16.0, 0.0, 8.0, 16.0]]
    g = np.random.default_rng(8)
    ids = g.integers(0, S, size=40).astype(np.int32)
    w = make_slices(61, 40, 256, [256, 136], S, ranks, alphas, ids, dtype="f32", r_max=8)
    ys, _, _ = run_multi(w)
    check_slices(w, ys, "f32 slices")


def test_unaligned_width_slices():
    """bf16 pools with d_in % 8 != 0 run the element-generic kernels slice
    after slice."""
    S = 4
    ranks = [[0, 8, 5, 8], [0, 3, 0, 8]]
    alphas = [[2.0 * r for r in rk] for rk in ranks]
    ids = np.random.default_rng(9).integers(0, S, size=90).astype(np.int32)
    w = make_slices(62, 90, 515, [200, 72], S, ranks, alphas, ids, r_max=8)
    ys, _, _ = run_multi(w)
    check_slices(w, ys, "unaligned slices")


def test_multi_argument_errors():
    """Pools that cannot share a call, aliasing outputs and a short workspace
    are refused before any launch."""
    L = lora.lib()
    a = lora.Pool(5, 16, 256, 128, "bf16")
    b = lora.Pool(5, 8, 256, 128, "bf16")
    c = lora.Pool(5, 16, 256, 64, "bf16")
    ids = np.array([0, 1, 2, 3], np.int32)
    p = lora.plan(ids, 5)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    Wa = torch.zeros((128, 256), dtype=torch.bfloat16, device="cuda")
    Wc = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    ya = torch.zeros((4, 128), dtype=torch.bfloat16, device="cuda")
    yc = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lora.LoraError) as e:
        lora.linear_multi(x, [Wa, Wa], [a, b], p, ys=[ya, ya.clone()], workspace=a.workspace(4))
    assert e.value.status == lora.LORA_EINVAL
    with pytest.raises(lora.LoraError) as e:
        lora.linear_multi(x, [Wa, Wa], [a, a], p, ys=[ya, ya], workspace=a.workspace(4))
    assert e.value.status == lora.LORA_EINVAL
    need = lora.workspace_bytes_multi([a, c], 4)
    assert need > 0 and lora.workspace_bytes_multi([a, b], 4) == 0
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(lora.LoraError) as e:
        lora.linear_multi(x, [Wa, Wc], [a, c], p, ys=[ya, yc], workspace=short)
    assert e.value.status == lora.LORA_ESPACE
    arr = (lora.SliceDesc * 5)()
    for i in range(5):
        arr[i].pool, arr[i].W, arr[i].y = a.handle, Wa.data_ptr(), ya.data_ptr() + i
    info = p.info
    to, ip, wk = p.dev_ptrs()
    assert L.lora_linear_multi(arr, 5, x.data_ptr(), to, ip, wk, ctypes.byref(info), 1, 1 << 30, None) \
        == lora.LORA_EINVAL
