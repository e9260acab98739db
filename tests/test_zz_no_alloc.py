"""lora_linear_noalloc (workspace in the library's own device array) against
lora_linear with a caller workspace, through the C ABI: the same kernels on
the same inputs give the same bits, and both match the fp64 oracle. Two
calls in a row, the second with a smaller input, so the array holds the
first call's contents when the second starts."""
import ctypes

import numpy as np
import pytest
import torch

from rank_gemm_amd import lora
from rank_gemm_amd.inputs import make_config, make_custom

from gpu_util import build_pool, check_close, oracle_pair, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    lora.lib()
    yield


def _noalloc(x, W, pool, p, y):
    to, ip, wk = p.dev_ptrs()
    rc = lora.lib().lora_linear_noalloc(pool.handle, x.data_ptr(), W.data_ptr(), to, ip, wk, ctypes.byref(p.info),
                                        y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return rc


def _case(w, proj):
    pool = build_pool(w, proj)
    x = lora.to_device(proj.x, w.dtype)
    W = lora.to_device(proj.W, w.dtype)
    p = lora.plan(w.slot_ids, w.S)
    need = pool.workspace_bytes(w.T)
    print(f"[noalloc] {w.name[:40]} T={w.T} workspace {need} bytes", flush=True)
    assert need <= lora.LORA_NOALLOC_MAX_WORKSPACE
    y_ref = lora.linear(x, W, pool, p, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    y = torch.full_like(y_ref, float("nan"))
    assert _noalloc(x, W, pool, p, y) == lora.LORA_OK
    torch.cuda.synchronize()
    bits = torch.int16 if w.dtype == "bf16" else torch.int32
    assert torch.equal(y.view(bits), y_ref.view(bits))
    ref, base = oracle_pair(w, proj)
    check_close(to_f64(y), ref, w.dtype, f"noalloc {w.name[:30]} T={w.T}", base if w.dtype == "bf16" else None)


def test_noalloc_two_calls_second_smaller():
    big = make_config(4)  # T = 256, r_max 64, 33 slots: split-K decode path with shrink tiles
    _case(big, big.projections[0])
    ids = np.random.default_rng(4).integers(0, 5, size=37).astype(np.int32)
    small = make_custom(45, 37, 4096, 1000, 5, [0, 16, 8, 0, 16], [0, 32, 16, 0, 32], ids, r_max=16)
    _case(small, small.projections[0])


def test_noalloc_prefill_then_decode():
    """A prefill-sized call (tiled path) then a decode-sized one (split-K)."""
    g = np.random.default_rng(8)
    ids = np.repeat(g.integers(0, 9, size=8), 256).astype(np.int32)
    pre = make_custom(46, 2048, 1024, 3000, 9, [0] + [16] * 8, [0] + [32.0] * 8, ids, r_max=16)
    _case(pre, pre.projections[0])
    dec = make_config(2)
    _case(dec, dec.projections[0])


def test_noalloc_refuses_oversized_workspace():
    """A call whose workspace would exceed the array is refused before any
    launch (the device pointers are never touched)."""
    T = 1 << 20
    pool = lora.Pool(3, 64, 4096, 64, "bf16")
    assert pool.workspace_bytes(T) > lora.LORA_NOALLOC_MAX_WORKSPACE
    info = lora.PlanInfo(T, 3, T, 1, 1, T, lora.LORA_PLAN_ROWS)
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    rc = lora.lib().lora_linear_noalloc(pool.handle, dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                        dummy.data_ptr(), dummy.data_ptr(), ctypes.byref(info), dummy.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    assert rc == lora.LORA_ESPACE
