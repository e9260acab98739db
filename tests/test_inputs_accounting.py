"""The seeded workload generator and the FLOP/byte accounting (CPU only).

Accounting is pinned to the closed forms of "LoRA serving, embeddings,
rerankers, pooling" (mlinterviewnotes.com): section "Adapter size" (one
adapter costs r*(d_in+d_out) parameters; 41.9 M for rank 16 over seven
Llama-3-8B targets; exactly r*5 MiB in bf16; attention-only sum 26,624,
13.63 M, 26 MiB) and the 0.78 % FLOP share of a rank-16 correction on a
square 4096 projection.
"""
import numpy as np
import pytest
import torch

from rank_gemm_amd import accounting as acc
from rank_gemm_amd.inputs import bf16_bits, bf16_to_f32, make_config, make_custom


def test_bf16_rne_matches_torch():
    g = np.random.default_rng(0)
    a = g.standard_normal(100000).astype(np.float32) * 10.0
    # exact ties: low 16 bits == 0x8000, both parities of the kept bit
    ties = (np.arange(64, dtype=np.uint32) << 17 | 0x3F800000 | 0x8000).view(np.float32)
    ties2 = (np.arange(64, dtype=np.uint32) << 17 | 0x3F810000 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, ties2, -ties])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits(a), want)
    np.testing.assert_array_equal(bf16_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_closed_forms():
    assert acc.adapter_params(16, 4096, 4096) == 16 * 8192
    assert acc.layer_width_sum() == 81920
    assert acc.model_adapter_params(16) == 41_943_040  # "41.9 M"
    for r in (1, 8, 16, 64):
        assert acc.model_adapter_bytes(r) == r * 5 * 2**20  # "exactly r*5 MiB"
    assert acc.layer_width_sum(acc.ATTENTION_TARGETS) == 26_624
    assert round(acc.model_adapter_params(16, acc.ATTENTION_TARGETS) / 1e6, 2) == 13.63
    assert acc.model_adapter_bytes(16, acc.ATTENTION_TARGETS) == 26 * 2**20
    assert acc.correction_to_base_ratio(16, 4096, 4096) == 0.0078125  # "0.78%"


def test_decode_bytes_closed_form():
    # q_proj decode, 8 adapters x 8 tokens, rank 16, bf16:
    # x rows 64*4096*2 + A,B 8*16*8192*2 + h 2*4*64*16 + y rmw 2*2*64*4096
    slot_ids = np.repeat(np.arange(1, 9), 8)
    ranks = np.array([0] + [16] * 8)
    assert acc.correction_bytes(slot_ids, ranks, 4096, 4096, 2, 16) == 3_678_208
    assert acc.base_flops(8192, 4096, 14336) == 962_072_674_304


def test_config_readings_small():
    w1 = make_config(1)
    assert w1.dtype == "f32" and w1.T == 64 and w1.S == 5 and w1.r_max == 8
    p = w1.projections[0]
    assert p.x.dtype == np.float32 and p.x.shape == (64, 256) and p.W.shape == (256, 256)
    assert sorted(p.adapters) == [1, 2, 3, 4] and all(a.rank == 8 and a.alpha == 16 for a in p.adapters.values())
    assert w1.slot_ids.min() >= 0 and w1.slot_ids.max() <= 4
    bound = 1 / np.sqrt(256)
    assert np.all(np.abs(p.adapters[1].A) <= bound)

    w2 = make_config(2)
    assert np.array_equal(np.bincount(w2.slot_ids), [0] + [8] * 8)
    assert w2.projections[0].x.dtype == np.uint16

    w4 = make_config(4)
    assert (w4.slot_ids == 0).sum() == 51
    ranks = w4.ranks
    assert ranks[0] == 0 and set(ranks[1:].tolist()) <= {8, 16, 32, 64}
    assert all(a.alpha == 2 * a.rank for a in w4.projections[0].adapters.values())
    assert w4.r_max == 64
    # Zipf(1.1): slot 1 is the most popular
    c = np.bincount(w4.slot_ids, minlength=33)
    assert c[1] == c[1:].max()


def test_configs_are_reproducible():
    a, b = make_config(1), make_config(1)
    assert np.array_equal(a.slot_ids, b.slot_ids)
    assert np.array_equal(a.projections[0].W, b.projections[0].W)
    c = make_config(1, layer=1)
    assert np.array_equal(a.slot_ids, c.slot_ids) and not np.array_equal(a.projections[0].W, c.projections[0].W)


@pytest.mark.slow
def test_config_readings_large():
    w3 = make_config(3)
    assert w3.T == 8192 and len(w3.projections) == 2
    seq = w3.slot_ids.reshape(16, 512)
    assert np.all(seq == seq[:, :1])
    assert w3.projections[0].x is w3.projections[1].x
    assert w3.projections[0].W.shape == (14336, 4096)
    w5 = make_config(5)
    assert len(np.unique(w5.slot_ids)) <= 50 and w5.slot_ids.min() >= 1
    assert [p.d_in for p in w5.projections] == [4096, 14336]
    assert len(w5.projections[1].adapters) == 128


def test_custom():
    w = make_custom(0, 37, 24, 9, 4, [0, 2, 0, 3], [0, 4, 0, 3], np.arange(37) % 4, dtype="bf16")
    assert w.r_max == 3 and sorted(w.projections[0].adapters) == [1, 3]
