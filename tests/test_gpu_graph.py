"""lora_linear captured in a HIP graph, the way the decode benchmark replays it.

Each replay must give, bit for bit, the outputs of the same calls made
eagerly: first with the plan the graph was captured with, then after the
device plan buffer is rewritten (plan_into) with another token-to-slot
assignment that has the same segment counts. Replays are separated by
eager work and synchronisations, so a graph node that only behaves on its
first replay would show up here.
"""

import numpy as np
import pytest

from rank_gemm_amd import lora
from rank_gemm_amd.inputs import make_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import build_pool  # noqa: E402

LAYERS = 4


def _setup():
    ws_list = [make_config(2, layer=l) for l in range(LAYERS)]
    w0 = ws_list[0]
    T = w0.T
    pools, xs, Ws, ys = [], [], [], []
    for w in ws_list:
        pr = w.projections[0]
        pools.append(build_pool(w, pr))
        xs.append(lora.to_device(pr.x, "bf16"))
        Ws.append(lora.to_device(pr.W, "bf16"))
        ys.append(torch.empty((T, pr.d_out), dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty(pools[0].workspace_bytes(T), dtype=torch.uint8, device="cuda")
    return w0, pools, xs, Ws, ys, ws


def test_graph_replay_matches_eager():
    w0, pools, xs, Ws, ys, ws = _setup()
    ids = w0.slot_ids.copy()
    p = lora.plan(ids, w0.S)

    def layers_once():
        for l in range(LAYERS):
            lora.linear(xs[l], Ws[l], pools[l], p, y=ys[l], workspace=ws)

    def eager(plan_ids):
        lora.plan_into(p, plan_ids)
        layers_once()
        torch.cuda.synchronize()
        return [y.clone() for y in ys]

    ref = eager(ids)
    # another assignment with the same segment counts: the captured launches
    # (grid sizes, item counts) stay valid for it
    rng = np.random.default_rng(5)
    ids2 = rng.permutation(ids).astype(np.int32)
    ref2 = eager(ids2)
    assert any(not torch.equal(a, b) for a, b in zip(ref, ref2))

    lora.plan_into(p, ids)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layers_once()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layers_once()
    torch.cuda.synchronize()

    filler = torch.randn(1024, 1024, device="cuda")
    for rep, (plan_ids, want) in enumerate([(ids, ref), (ids, ref), (ids2, ref2), (ids, ref)]):
        for y in ys:
            y.fill_(float("nan"))
        lora.plan_into(p, plan_ids)
        graph.replay()
        filler = filler @ filler * 1e-3  # eager work between replays
        torch.cuda.synchronize()
        for l in range(LAYERS):
            assert torch.equal(ys[l], want[l]), f"replay {rep} layer {l} differs from the eager call"
