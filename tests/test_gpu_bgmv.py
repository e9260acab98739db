"""The BGMV shrink (token by token, no plan) against the oracle's h and the
SGMV shrink: the same values to fp32 rounding (another summation order)."""
import numpy as np
import pytest
import torch

from rank_gemm_amd import lora
from rank_gemm_amd.inputs import make_config, make_custom

from gpu_util import build_pool, oracle_rows, rel_err, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    lora.lib()
    yield


def run_both(w, proj, ids=None):
    ids = w.slot_ids if ids is None else ids
    pool = build_pool(w, proj)
    x = lora.to_device(proj.x, w.dtype)
    h_b = to_f64(lora.shrink_bgmv(x, pool, torch.from_numpy(np.asarray(ids, np.int32)).cuda()))
    h_s = to_f64(lora.shrink(x, pool, lora.plan(ids, w.S)))
    torch.cuda.synchronize()
    return h_b, h_s


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_bgmv_h_matches_oracle_and_sgmv(cfg):
    w = make_config(cfg)
    proj = w.projections[0]
    rows = None if w.T <= 512 else np.arange(0, w.T, 37, dtype=np.int32)
    h_b, h_s = run_both(w, proj)
    _, h_ref = oracle_rows(w, proj, rows=rows, want_h=True)
    sel = slice(None) if rows is None else rows
    e_b, e_s = rel_err(h_b[sel], h_ref), rel_err(h_s[sel], h_ref)
    print(f"[bgmv] config {cfg}: bgmv rel_err={e_b:.2e} sgmv rel_err={e_s:.2e}", flush=True)
    assert e_b <= 1e-4 and e_s <= 1e-4
    assert rel_err(h_b, h_s) <= 1e-5
    assert np.all(h_b[w.slot_ids == 0] == 0)


def test_bgmv_ragged_ranks_and_invalid_ids():
    S = 6
    g = np.random.default_rng(21)
    ids = g.integers(0, S, size=45).astype(np.int32)
    w = make_custom(5, 45, 1032, 64, S, [0, 80, 17, 0, 64, 3], [0, 160, 34, 0, 128, 6], ids, r_max=80)
    proj = w.projections[0]
    h_b, h_s = run_both(w, proj)
    _, h_ref = oracle_rows(w, proj, want_h=True)
    assert rel_err(h_b, h_ref) <= 1e-4
    assert rel_err(h_b, h_s) <= 1e-5
    bad = ids.copy()
    bad[:5] = [-1, S, 99, -7, S + 1]
    pool = build_pool(w, proj)
    hb = lora.shrink_bgmv(lora.to_device(proj.x, "bf16"), pool, torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    assert torch.count_nonzero(hb[:5]) == 0
