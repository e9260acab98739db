"""The device planner and lora_linear over a device plan.

The device plan must equal lora_plan's bit for bit (token order, CSR
offsets, work list, summary) with its work list padded by empty items; the
layer over it must match the oracle, and on the decode path the host-plan
call bit for bit. A graph that captures the planner and the layers once must
follow any new token-to-slot assignment written into the captured id buffer.
"""
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


def check_same_plan(ids, S, clamp=False):
    dev = lora.plan_device(torch.from_numpy(np.asarray(ids, np.int32)).cuda(), S)
    d = dev.read()
    ref_ids = np.where((ids < 0) | (ids >= S), 0, ids).astype(np.int32) if clamp else ids
    h = lora.plan(ref_ids, S, upload=False)
    np.testing.assert_array_equal(d["token_order"], h.token_order)
    np.testing.assert_array_equal(d["slot_indptr"], h.slot_indptr)
    np.testing.assert_array_equal(d["work"], h.work)
    assert (d["pad"] == 0).all()
    for k in ("T", "S", "T_a", "k", "n_items", "max_seg"):
        assert d[k] == getattr(h.info, k), k
    return d


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_device_plan_matches_host_on_configs(cfg):
    w = make_config(cfg)
    d = check_same_plan(w.slot_ids, w.S)
    assert d["status"] == lora.LORA_OK


@pytest.mark.parametrize("T,S,kind", [(0, 5, "uniform"), (1, 2, "uniform"), (63, 9, "uniform"), (65, 9, "zipf"),
                                      (1000, 129, "uniform"), (4097, 1025, "uniform"), (3000, 4096, "zipf"),
                                      (8192, 17, "runs"), (777, 3, "base")])
def test_device_plan_matches_host_random(T, S, kind):
    g = np.random.default_rng(T * 7 + S)
    if kind == "uniform":
        ids = g.integers(0, S, size=T)
    elif kind == "zipf":
        p = np.arange(1, S + 1, dtype=np.float64) ** -1.1
        ids = g.choice(S, size=T, p=p / p.sum())
    elif kind == "runs":
        ids = np.repeat(g.integers(0, S, size=16), T // 16)
    else:
        ids = np.zeros(T)
    check_same_plan(ids.astype(np.int32), S)


def test_device_plan_invalid_ids_are_base_rows():
    ids = np.array([1, 2, -1, 2, 5, 0, 1, 7, 3], np.int32)
    d = check_same_plan(ids, 5, clamp=True)
    assert d["status"] == lora.LORA_ESLOT


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_linear_over_device_plan(cfg):
    """Oracle parity; on the decode path also bit-equal to the host-plan call."""
    w = make_config(cfg)
    proj = w.projections[0]
    pool = build_pool(w, proj)
    x, W = lora.to_device(proj.x, w.dtype), lora.to_device(proj.W, w.dtype)
    dp = lora.plan_device(torch.from_numpy(w.slot_ids).cuda(), w.S)
    y = torch.full((w.T, proj.d_out), float("nan"), dtype=x.dtype, device="cuda")
    y = lora.linear(x, W, pool, dp, y=y)
    y_host = lora.linear(x, W, pool, lora.plan(w.slot_ids, w.S))
    torch.cuda.synchronize()
    ref, base = oracle_pair(w, proj)
    check_close(to_f64(y), ref, w.dtype, f"config {cfg} device plan", base if w.dtype == "bf16" else None)
    if w.dtype == "bf16":
        assert torch.equal(y.view(torch.int16), y_host.view(torch.int16))


def test_linear_over_device_plan_tiled_and_base_only():
    S = 6
    g = np.random.default_rng(4)
    ids = np.repeat(g.integers(0, S, size=20), 100).astype(np.int32)
    w = make_custom(9, 2000, 512, 2048, S, [0, 16, 8, 0, 16, 4], [0, 32, 16, 0, 32, 8], ids, r_max=16)
    proj = w.projections[0]
    pool = build_pool(w, proj)
    x, W = lora.to_device(proj.x, "bf16"), lora.to_device(proj.W, "bf16")
    y = lora.linear(x, W, pool, lora.plan_device(torch.from_numpy(ids).cuda(), S))
    torch.cuda.synchronize()
    ref, base = oracle_pair(w, proj)
    check_close(to_f64(y), ref, "bf16", "tiled, device plan", base)
    zeros = np.zeros_like(ids)
    y0 = lora.linear(x, W, pool, lora.plan_device(torch.from_numpy(zeros).cuda(), S))
    y0h = lora.linear(x, W, pool, lora.plan(zeros, S))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y0h.view(torch.int16))
    rows = torch.from_numpy(ids == 0).cuda()
    assert torch.equal(y[rows].view(torch.int16), y0h[rows].view(torch.int16))


def test_graph_with_device_plan_follows_new_assignments():
    """Planner + 4 decode layers captured once; each replay after writing new
    ids (other segment counts each time) equals the eager host-plan calls."""
    LAYERS = 4
    ws_list = [make_config(2, layer=l) for l in range(LAYERS)]
    w0 = ws_list[0]
    T, S = w0.T, w0.S
    pools, xs, Ws, ys = [], [], [], []
    for w in ws_list:
        pr = w.projections[0]
        pools.append(build_pool(w, pr))
        xs.append(lora.to_device(pr.x, "bf16"))
        Ws.append(lora.to_device(pr.W, "bf16"))
        ys.append(torch.empty((T, pr.d_out), dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty(pools[0].workspace_bytes(T), dtype=torch.uint8, device="cuda")
    ids_dev = torch.from_numpy(w0.slot_ids.copy()).cuda()
    dp = lora.plan_device(ids_dev, S)

    def step():
        lora.plan_device(ids_dev, S, out=dp)
        for l in range(LAYERS):
            lora.linear(xs[l], Ws[l], pools[l], dp, y=ys[l], workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    g = np.random.default_rng(12)
    assignments = [w0.slot_ids, np.zeros(T, np.int32), g.integers(0, S, size=T).astype(np.int32),
                   np.full(T, 3, np.int32), g.permutation(np.repeat(np.arange(1, 5), 16)).astype(np.int32)]
    filler = torch.randn(512, 512, device="cuda")
    for rep, ids in enumerate(assignments):
        p = lora.plan(ids, S)
        want = [lora.linear(xs[l], Ws[l], pools[l], p) for l in range(LAYERS)]
        torch.cuda.synchronize()
        for y in ys:
            y.fill_(float("nan"))
        ids_dev.copy_(torch.from_numpy(ids))
        graph.replay()
        filler = filler @ filler * 1e-3
        torch.cuda.synchronize()
        for l in range(LAYERS):
            assert torch.equal(ys[l].view(torch.int16), want[l].view(torch.int16)), f"assignment {rep} layer {l}"


def test_multi_slice_over_device_plan_in_a_graph():
    """q/k/v in one lora_linear_multi_device_plan call, planner and call
    captured once; replays after new assignments equal the host-plan call."""
    from rank_gemm_amd.inputs import make_qkv_decode

    w = make_qkv_decode()
    T, S = w.T, w.S
    pools = [build_pool(w, pr) for pr in w.projections]
    x = lora.to_device(w.projections[0].x, "bf16")
    Ws = [lora.to_device(pr.W, "bf16") for pr in w.projections]
    ys = [torch.empty((T, pr.d_out), dtype=torch.bfloat16, device="cuda") for pr in w.projections]
    ws = torch.empty(lora.workspace_bytes_multi(pools, T), dtype=torch.uint8, device="cuda")
    ids_dev = torch.from_numpy(w.slot_ids.copy()).cuda()
    dp = lora.plan_device(ids_dev, S)

    def step():
        lora.plan_device(ids_dev, S, out=dp)
        lora.linear_multi(x, Ws, pools, dp, ys=ys, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    for rep, ids in enumerate([w.slot_ids, g.integers(0, S, size=T).astype(np.int32), np.zeros(T, np.int32)]):
        want = lora.linear_multi(x, Ws, pools, lora.plan(ids, S))
        torch.cuda.synchronize()
        for y in ys:
            y.fill_(float("nan"))
        ids_dev.copy_(torch.from_numpy(ids))
        graph.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(ys[i].view(torch.int16), want[i].view(torch.int16)), f"assignment {rep} slice {i}"


@pytest.mark.parametrize("words", [1, 3, 4, 5, 1027, 40_013])
def test_plan_upload_kernel(words):
    """lora_plan_upload copies a pinned host buffer bit for bit, at word
    counts that take the 16-byte path with and without tail words and the
    word path (an unaligned source); pageable host memory is refused."""
    L = lora.lib()
    g = np.random.default_rng(words)
    host = torch.from_numpy(g.integers(-2**31, 2**31 - 1, size=words + 1, dtype=np.int64).astype(np.int32)).pin_memory()
    for off in (0, 1):  # off = 1: a source 4 bytes past 16-byte alignment
        n = words - off if words > off else words
        dev = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        rc = L.lora_plan_upload(host.data_ptr() + 4 * off, dev.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
        assert rc == lora.LORA_OK
        torch.cuda.synchronize()
        assert torch.equal(dev.cpu(), host[off:off + n])
    pageable = np.arange(words, dtype=np.int32)
    dev = torch.empty(words, dtype=torch.int32, device="cuda")
    assert L.lora_plan_upload(pageable.ctypes.data, dev.data_ptr(), words, None) == lora.LORA_EINVAL


def test_plan_into_steps_follow_new_ids():
    """plan_into over many steps (the two pinned staging buffers in turn, each
    uploaded by the kernel) gives each step's plan bit for bit."""
    g = np.random.default_rng(7)
    T, S = 1000, 17
    p = lora.plan(g.integers(0, S, size=T).astype(np.int32), S)
    for step in range(6):
        ids = g.integers(0, S, size=T).astype(np.int32)
        lora.plan_into(p, ids)
        ref = lora.plan(ids, S, upload=False)
        torch.cuda.synchronize()
        got = p.dev.cpu().numpy()
        nw, ni = p._n_work, ref.info.n_items
        assert p.info.n_items == ni
        np.testing.assert_array_equal(got[4 * nw:4 * nw + T], ref.token_order)
        np.testing.assert_array_equal(got[4 * nw + T:4 * nw + T + S + 1], ref.slot_indptr)
        np.testing.assert_array_equal(got[:4 * ni].reshape(ni, 4)[:, :3], ref.work[:, :3])
