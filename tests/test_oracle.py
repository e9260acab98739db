"""Pins of the fp64 CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: hand-derived outputs, the merged-weight identity, closed forms, the
base-only invariant of slot 0, textbook special cases and exact rational
arithmetic on tiny inputs.
"""
import fractions

import numpy as np
import pytest

import oracle
from rank_gemm_amd.inputs import Adapter, bf16_bits, bf16_to_f32

FORMS = ("rows", "merged", "grouped")


def run_form(form, dtype, x, W, S, adapters, slot_ids):
    if form == "rows":
        return oracle.lora_rows(dtype, x, W, S, adapters, slot_ids)
    if form == "merged":
        return oracle.lora_merged(dtype, x, W, S, adapters, slot_ids)
    return oracle.lora_grouped(dtype, x, W, S, adapters, slot_ids)


def enc(a, dtype):
    a = np.asarray(a, np.float32)
    return bf16_bits(a) if dtype == "bf16" else a


def hand_case(g, name, dtype):
    sec = g("hand_examples.txt")[name]
    d_in, d_out, S = int(sec["d_in"][0]), int(sec["d_out"][0]), int(sec["S"][0])
    x = np.atleast_2d(sec["x"]).reshape(-1, d_in)
    W = np.atleast_2d(sec["W"]).reshape(d_out, d_in)
    ads = {}
    for s in range(1, S):
        r = int(sec["rank"][s])
        if r:
            A = np.asarray(sec[f"A{s}"]).reshape(r, d_in)
            B = np.asarray(sec[f"B{s}"]).reshape(d_out, r)
            ads[s] = Adapter(r, float(sec["alpha"][s]), enc(A, dtype), enc(B, dtype))
    slot_ids = sec["slot_ids"].astype(np.int32)
    y = np.atleast_2d(sec["y"]).reshape(len(slot_ids), d_out)
    h = np.atleast_2d(sec["h"]).reshape(len(slot_ids), -1)
    return enc(x, dtype), enc(W, dtype), S, ads, slot_ids, y, h


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("name", ["H1", "H2"])
def test_hand_examples(golden, name, form, dtype):
    x, W, S, ads, slot_ids, y_ref, _ = hand_case(golden, name, dtype)
    y = run_form(form, dtype, x, W, S, ads, slot_ids)
    np.testing.assert_array_equal(y, y_ref)


@pytest.mark.parametrize("name", ["H1", "H2"])
def test_hand_examples_h(golden, name):
    x, W, S, ads, slot_ids, _, h_ref = hand_case(golden, name, "f32")
    _, h = oracle.lora_rows("f32", x, W, S, ads, slot_ids, want_h=True, h_width=h_ref.shape[1])
    np.testing.assert_array_equal(h, h_ref)


def test_page_merged_parity_check():
    """The merged-parity check printed on the mlinterviewnotes page
    (default_rng(5), x 3x4, w 6x4, a 2x4, b 6x2, scale 0.5, atol 1e-12):
    the oracle's unmerged rows must equal x @ (w + scale*b@a).T, the merged
    form evaluated by numpy. fp32 copies of the draws are used, since the
    oracle takes fp32 or bf16 inputs; the identity is exact either way."""
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 4)).astype(np.float32)
    w = rng.normal(size=(6, 4)).astype(np.float32)
    a = rng.normal(size=(2, 4)).astype(np.float32)
    b = rng.normal(size=(6, 2)).astype(np.float32)
    scale = 0.5  # alpha / r with r = 2 -> alpha = 1
    ads = {1: Adapter(2, 1.0, a, b)}
    slot_ids = np.ones(3, np.int32)
    y = oracle.lora_rows("f32", x, w, 2, ads, slot_ids)
    X, Wd, A, B = (v.astype(np.float64) for v in (x, w, a, b))
    merged = X @ (Wd + scale * B @ A).T
    np.testing.assert_allclose(y, merged, atol=1e-12, rtol=0)


def random_case(seed, T, d_in, d_out, S, ranks, dtype, p0=0.25):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, d_in)).astype(np.float32)
    W = (0.3 * g.standard_normal((d_out, d_in))).astype(np.float32)
    ads = {}
    for s in range(1, S):
        r = int(ranks[s])
        if r:
            ads[s] = Adapter(r, float(g.choice([r, 2 * r, 0.5 * r])),
                             enc(g.uniform(-1, 1, (r, d_in)), dtype), enc(0.5 * g.standard_normal((d_out, r)), dtype))
    slot_ids = g.integers(1, S, size=T).astype(np.int32)
    slot_ids[g.random(T) < p0] = 0
    return enc(x, dtype), enc(W, dtype), ads, slot_ids


def as_f64(a, dtype):
    return (bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forms_agree_mixed_ranks(dtype):
    """Per-row, merged and grouped forms agree on mixed ranks, empty slots and
    base rows (mlinterviewnotes merged identity; shantanugoel grouped form)."""
    S, ranks = 6, [0, 3, 1, 0, 5, 2]
    x, W, ads, slot_ids = random_case(11, 29, 13, 7, S, ranks, dtype)
    ys = [run_form(f, dtype, x, W, S, ads, slot_ids) for f in FORMS]
    scale = np.max(np.abs(ys[0]))
    for y in ys[1:]:
        assert np.max(np.abs(y - ys[0])) <= 1e-12 * scale


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merged_form_numpy(dtype):
    """Rows of the oracle equal the merged weight applied by numpy's matmul:
    y_i = (W + scale_s B_s A_s) x_i, one slot at a time."""
    S, ranks = 5, [0, 4, 2, 1, 3]
    x, W, ads, slot_ids = random_case(3, 40, 24, 9, S, ranks, dtype)
    y = oracle.lora_rows(dtype, x, W, S, ads, slot_ids)
    X, Wd = as_f64(x, dtype), as_f64(W, dtype)
    for i, s in enumerate(slot_ids):
        Wp = Wd.copy()
        if s:
            a = ads[s]
            Wp += (a.alpha / a.rank) * as_f64(a.B, dtype) @ as_f64(a.A, dtype)
        np.testing.assert_allclose(y[i], Wp @ X[i], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_slot0_rows_are_exact_base(dtype):
    """Rows on slot 0 get exactly the base output (mstar pool: the zero
    adapter, rank 0, scaling 0); base = x W^T by numpy within rounding."""
    S, ranks = 4, [0, 2, 3, 1]
    x, W, ads, slot_ids = random_case(5, 50, 16, 12, S, ranks, dtype, p0=0.4)
    y = oracle.lora_rows(dtype, x, W, S, ads, slot_ids)
    y0 = oracle.lora_rows(dtype, x, W, S, ads, np.zeros_like(slot_ids))
    base_rows = slot_ids == 0
    assert base_rows.any() and (~base_rows).any()
    np.testing.assert_array_equal(y[base_rows], y0[base_rows])
    np.testing.assert_allclose(y0, as_f64(x, dtype) @ as_f64(W, dtype).T, rtol=1e-13, atol=1e-13)
    assert np.all(np.abs(y[~base_rows] - y0[~base_rows]).max(axis=1) > 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_base_output_equals_all_slot0_run(dtype):
    """The base term returned beside y (want_base) is, bit for bit, the y of a
    run where every row is on slot 0, and it equals numpy's x W^T within
    rounding; y itself is unchanged by asking for it."""
    S, ranks = 4, [0, 2, 3, 1]
    x, W, ads, slot_ids = random_case(15, 33, 16, 12, S, ranks, dtype, p0=0.3)
    y_alone = oracle.lora_rows(dtype, x, W, S, ads, slot_ids)
    y, base = oracle.lora_rows(dtype, x, W, S, ads, slot_ids, want_base=True)
    np.testing.assert_array_equal(y, y_alone)
    np.testing.assert_array_equal(base, oracle.lora_rows(dtype, x, W, S, ads, np.zeros_like(slot_ids)))
    np.testing.assert_allclose(base, as_f64(x, dtype) @ as_f64(W, dtype).T, rtol=1e-13, atol=1e-13)
    rows = np.array([0, 5, 32, 7], np.int32)
    y_r, h_r, base_r = oracle.lora_rows(dtype, x, W, S, ads, slot_ids, rows=rows, want_h=True, h_width=3,
                                        want_base=True)
    np.testing.assert_array_equal(y_r, y[rows])
    np.testing.assert_array_equal(base_r, base[rows])


def test_rank1_closed_form():
    """A rank-1 adapter adds scale * (a . x) * b, an outer product."""
    x, W, _, _ = random_case(7, 9, 10, 6, 2, [0, 1], "f32")
    g = np.random.default_rng(8)
    a = g.standard_normal((1, 10)).astype(np.float32)
    b = g.standard_normal((6, 1)).astype(np.float32)
    ads = {1: Adapter(1, 3.0, a, b)}
    slots = np.ones(9, np.int32)
    d = oracle.lora_rows("f32", x, W, 2, ads, slots) - oracle.lora_rows("f32", x, W, 2, ads, 0 * slots)
    expect = 3.0 * np.outer(x.astype(np.float64) @ a[0].astype(np.float64), b[:, 0].astype(np.float64))
    np.testing.assert_allclose(d, expect, rtol=1e-12, atol=1e-12)


def test_zero_B_gives_base():
    x, W, ads, slot_ids = random_case(9, 20, 8, 8, 3, [0, 2, 2], "f32")
    for a in ads.values():
        a.B = np.zeros_like(a.B)
    y = oracle.lora_rows("f32", x, W, 3, ads, slot_ids)
    y0 = oracle.lora_rows("f32", x, W, 3, ads, np.zeros_like(slot_ids))
    np.testing.assert_array_equal(y, y0)


def test_exact_rational_brute_force():
    """Tiny bf16 case against exact rational arithmetic (fractions): the
    fp64 oracle must sit within a few ulps of the exact value."""
    S, ranks = 3, [0, 2, 1]
    x, W, ads, slot_ids = random_case(13, 6, 5, 4, S, ranks, "bf16", p0=0.3)
    y = oracle.lora_rows("bf16", x, W, S, ads, slot_ids)
    F = fractions.Fraction
    X = [[F(float(v)) for v in r] for r in bf16_to_f32(x)]
    Wf = [[F(float(v)) for v in r] for r in bf16_to_f32(W)]
    for i, s in enumerate(slot_ids):
        for j in range(W.shape[0]):
            val = sum(Wf[j][k] * X[i][k] for k in range(5))
            if s:
                a = ads[s]
                A = [[F(float(v)) for v in r] for r in bf16_to_f32(a.A)]
                B = [[F(float(v)) for v in r] for r in bf16_to_f32(a.B)]
                h = [sum(A[q][k] * X[i][k] for k in range(5)) for q in range(a.rank)]
                val += F(a.alpha) / a.rank * sum(B[j][q] * h[q] for q in range(a.rank))
            assert abs(float(val) - y[i, j]) <= 1e-14 * max(1.0, abs(float(val)))


def test_h_is_shrink_output():
    """h_i[q] = A_s[q] . x_i for q < r_s, zero-padded to the requested width."""
    S, ranks = 4, [0, 3, 1, 2]
    x, W, ads, slot_ids = random_case(21, 15, 12, 5, S, ranks, "f32")
    _, h = oracle.lora_rows("f32", x, W, S, ads, slot_ids, want_h=True, h_width=4)
    X = x.astype(np.float64)
    for i, s in enumerate(slot_ids):
        want = np.zeros(4)
        if s:
            want[: ads[s].rank] = ads[s].A.astype(np.float64) @ X[i]
        np.testing.assert_allclose(h[i], want, rtol=1e-13, atol=1e-13)


def test_row_subset_matches_full():
    S, ranks = 4, [0, 3, 1, 2]
    x, W, ads, slot_ids = random_case(22, 31, 16, 9, S, ranks, "bf16")
    full = oracle.lora_rows("bf16", x, W, S, ads, slot_ids)
    rows = np.array([30, 0, 7, 7, 12], np.int32)
    part = oracle.lora_rows("bf16", x, W, S, ads, slot_ids, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -133]
    np.testing.assert_array_equal(oracle.decode_bf16(bits), want)


def test_bad_slot_rejected():
    x, W, ads, slot_ids = random_case(1, 4, 8, 4, 2, [0, 1], "f32")
    slot_ids[2] = 2
    with pytest.raises(ValueError):
        oracle.lora_rows("f32", x, W, 2, ads, slot_ids)
    slot_ids[2] = -1
    with pytest.raises(ValueError):
        oracle.lora_grouped("f32", x, W, 2, ads, slot_ids)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_slot_is_two_textbook_gemms(dtype):
    """Every row on one slot: the layer is x W^T plus (alpha / r) (x A^T) B^T,
    written here as plain triple loops over Python floats (no numpy product),
    for all three oracle forms."""
    T, d_in, d_out, r, alpha = 5, 6, 4, 3, 1.5
    g = np.random.default_rng(31)
    x = enc(g.standard_normal((T, d_in)), dtype)
    W = enc(g.standard_normal((d_out, d_in)), dtype)
    A = enc(g.standard_normal((r, d_in)), dtype)
    B = enc(g.standard_normal((d_out, r)), dtype)
    dec = (lambda a: bf16_to_f32(a).astype(float)) if dtype == "bf16" else (lambda a: np.asarray(a, float))
    xf, Wf, Af, Bf = (dec(a).tolist() for a in (x, W, A, B))
    y = [[0.0] * d_out for _ in range(T)]
    for i in range(T):
        h = [sum(xf[i][k] * Af[q][k] for k in range(d_in)) for q in range(r)]
        for j in range(d_out):
            base = sum(xf[i][k] * Wf[j][k] for k in range(d_in))
            y[i][j] = base + (alpha / r) * sum(h[q] * Bf[j][q] for q in range(r))
    ads = {1: Adapter(r, alpha, A, B)}
    for form in FORMS:
        got = run_form(form, dtype, x, W, 2, ads, np.ones(T, np.int32))
        np.testing.assert_allclose(got, np.array(y), rtol=1e-12, atol=1e-12, err_msg=form)
