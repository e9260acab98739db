"""liblora on the CPU: the library loads, exports every symbol the header
declares, its host planner matches the oracle planner bit for bit, and its
host-side argument checks return the documented status codes. No kernel is
launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from rank_gemm_amd import lora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "lora.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_\w+)\s*\(", text)))


def test_exports_match_header():
    names = header_functions()
    assert set(names) == set(lora.EXPORTS)
    L = ctypes.CDLL(lora.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = lora.status_string(code)
        assert s and s != "unknown status"
    assert lora.status_string(42) == "unknown status"


def cpu_plan(ids, S):
    return lora.plan(ids, S, upload=False)


def test_plan_page_example(golden):
    g = golden("plan_worked_example.txt")[""]
    p = cpu_plan(g["slot_ids"].astype(np.int32), int(g["S"][0]))
    np.testing.assert_array_equal(p.token_order, g["token_order"].astype(np.int32))
    np.testing.assert_array_equal(p.slot_indptr, g["slot_indptr"].astype(np.int32))
    assert (p.info.T, p.info.S, p.info.T_a, p.info.k, p.info.n_items, p.info.max_seg) == (12, 3, 9, 2, 2, 5)
    assert p.work.tolist() == [[1, 3, 5, 0], [2, 8, 4, 0]]


@pytest.mark.parametrize("seed", range(40))
def test_plan_matches_oracle(seed):
    g = np.random.default_rng(seed)
    S = int(g.integers(1, 200))
    T = int(g.integers(0, 3000))
    if seed % 3 == 0:  # skewed, with long segments
        ids = np.minimum(g.zipf(1.3, size=T) - 1, S - 1).astype(np.int32)
    else:
        ids = g.integers(0, S, size=T).astype(np.int32)
    p = cpu_plan(ids, S)
    order, indptr, counts = oracle.plan(ids, S)
    np.testing.assert_array_equal(p.token_order, order)
    np.testing.assert_array_equal(p.slot_indptr, indptr)
    wl = oracle.work_list(indptr, lora.LORA_PLAN_ROWS)
    np.testing.assert_array_equal(p.work[:, :3], wl)
    assert np.all(p.work[:, 3] == 0)
    assert p.info.T_a == T - counts[0]
    assert p.info.k == int(np.count_nonzero(counts[1:]))
    assert p.info.n_items == len(wl)
    assert p.info.max_seg == int(counts[1:].max(initial=0))
    assert p.info.n_items <= lora.lib().lora_plan_max_items(T, S) or T == 0


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("seed", range(12))
def test_chunked_plan_matches_oracle(seed, chunk):
    """lora_plan_chunked: the same token order and CSR offsets as lora_plan,
    and the oracle's work list cut at `chunk` rows."""
    g = np.random.default_rng(1000 + seed)
    S = int(g.integers(1, 120))
    T = int(g.integers(0, 5000))
    ids = (np.minimum(g.zipf(1.1, size=T) - 1, S - 1) if seed % 2 else g.integers(0, S, size=T)).astype(np.int32)
    p = lora.plan(ids, S, upload=False, chunk=chunk)
    order, indptr, counts = oracle.plan(ids, S)
    np.testing.assert_array_equal(p.token_order, order)
    np.testing.assert_array_equal(p.slot_indptr, indptr)
    wl = oracle.work_list(indptr, chunk)
    np.testing.assert_array_equal(p.work[:, :3], wl)
    assert p.info.chunk == chunk and p.info.n_items == len(wl)
    assert p.info.n_items <= lora.lib().lora_plan_max_items(T, S) or T == 0


def test_chunked_plan_errors():
    L = lora.lib()
    info = lora.PlanInfo()
    ids = np.array([1, 2, 1], np.int32)
    out = np.zeros(64, np.int32)
    for bad in (0, 8, 24, 256):
        assert L.lora_plan_chunked(3, ids.ctypes.data, 3, bad, out.ctypes.data, out[8:].ctypes.data,
                                   out[16:].ctypes.data, 8, ctypes.byref(info)) == lora.LORA_EINVAL
    assert L.lora_plan(3, ids.ctypes.data, 3, out.ctypes.data, out[8:].ctypes.data, out[16:].ctypes.data, 8,
                       ctypes.byref(info)) == lora.LORA_OK
    assert info.chunk == lora.LORA_PLAN_ROWS


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_plan_configs(cfg):
    from rank_gemm_amd.inputs import make_config
    w = make_config(cfg)
    p = cpu_plan(w.slot_ids, w.S)
    order, indptr, _ = oracle.plan(w.slot_ids, w.S)
    np.testing.assert_array_equal(p.token_order, order)
    np.testing.assert_array_equal(p.slot_indptr, indptr)


def test_plan_errors():
    L = lora.lib()
    info = lora.PlanInfo()
    ids = np.array([0, 1, 5], np.int32)
    out = np.zeros(64, np.int32)
    # id out of range: rejected before any output is written
    out[:] = -7
    rc = L.lora_plan(3, ids.ctypes.data, 3, out.ctypes.data, out[8:].ctypes.data, out[16:].ctypes.data, 8,
                     ctypes.byref(info))
    assert rc == lora.LORA_ESLOT and np.all(out == -7)
    ids = np.array([0, -1], np.int32)
    assert L.lora_plan(3, ids.ctypes.data, 2, out.ctypes.data, out[8:].ctypes.data, out[16:].ctypes.data, 8,
                       ctypes.byref(info)) == lora.LORA_ESLOT
    ids = np.array([1, 2, 1], np.int32)
    assert L.lora_plan(3, ids.ctypes.data, 3, out.ctypes.data, out[8:].ctypes.data, out[16:].ctypes.data, 1,
                       ctypes.byref(info)) == lora.LORA_ESPACE
    assert L.lora_plan(0, ids.ctypes.data, 3, out.ctypes.data, out[8:].ctypes.data, out[16:].ctypes.data, 8,
                       ctypes.byref(info)) == lora.LORA_EINVAL
    assert L.lora_plan(3, ids.ctypes.data, -1, out.ctypes.data, out[8:].ctypes.data, out[16:].ctypes.data, 8,
                       ctypes.byref(info)) == lora.LORA_EINVAL


def test_plan_empty_and_base_only():
    p = cpu_plan(np.zeros(0, np.int32), 4)
    assert p.info.T == 0 and p.info.n_items == 0
    np.testing.assert_array_equal(p.slot_indptr, [0, 0, 0, 0, 0])
    p = cpu_plan(np.zeros(33, np.int32), 4)
    assert p.info.T_a == 0 and p.info.n_items == 0 and p.info.k == 0
    np.testing.assert_array_equal(p.token_order, np.arange(33))


def test_max_items_bound():
    L = lora.lib()
    for T, S in [(0, 5), (1, 2), (16, 2), (17, 2), (100, 9), (8192, 17), (5, 1000)]:
        bound = L.lora_plan_max_items(T, S)
        # worst case: every non-zero slot gets a ragged segment
        g = np.random.default_rng(T + S)
        for _ in range(20):
            ids = g.integers(0, S, size=T).astype(np.int32) if S > 1 else np.zeros(T, np.int32)
            p = cpu_plan(ids, S)
            assert p.info.n_items <= bound


def test_host_argument_errors():
    L = lora.lib()
    h = ctypes.c_void_p()
    # invalid shapes are refused before any HIP call
    assert L.lora_pool_create(ctypes.byref(h), 1, 16, 64, 64, 1, 1, 1, 1, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_create(ctypes.byref(h), 4, 0, 64, 64, 1, 1, 1, 1, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_create(ctypes.byref(h), 4, 16, 0, 64, 1, 1, 1, 1, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_create(ctypes.byref(h), 4, 16, 64, 0, 1, 1, 1, 1, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_create(ctypes.byref(h), 4, 16, 64, 64, 7, 1, 1, 1, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_create(ctypes.byref(h), 4, 16, 64, 64, 1, None, 1, 1, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_create(None, 4, 16, 64, 64, 1, 1, 1, 1, 1, None) == lora.LORA_EINVAL
    info = lora.PlanInfo()
    assert L.lora_linear(None, 1, 1, 1, 1, 1, ctypes.byref(info), 1, 1, 0, None) == lora.LORA_EINVAL
    assert L.lora_shrink(None, 1, 1, 1, 1, ctypes.byref(info), 1, 1, 0, None) == lora.LORA_EINVAL
    assert L.lora_pool_install(None, 1, 1, 1, 1, 1.0, None) == lora.LORA_EINVAL
    assert L.lora_pool_clear(None, 1, None) == lora.LORA_EINVAL
    assert L.lora_pool_rank(None, 0) == -1
    assert L.lora_workspace_bytes(None, 10) == 0


def test_plan_upload_argument_errors():
    """lora_plan_upload refuses null pointers and host memory the GPU cannot
    read (pageable numpy memory; here no GPU at all) before launching
    anything; zero words is a no-op."""
    L = lora.lib()
    buf = np.arange(64, dtype=np.int32)
    assert L.lora_plan_upload(None, 1, 64, None) == lora.LORA_EINVAL
    assert L.lora_plan_upload(buf.ctypes.data, None, 64, None) == lora.LORA_EINVAL
    assert L.lora_plan_upload(None, None, 0, None) == lora.LORA_OK
    assert L.lora_plan_upload(buf.ctypes.data, 1, 64, None) == lora.LORA_EINVAL


def test_multi_host_argument_errors():
    """lora_linear_multi refuses a missing slice array, a slice count outside
    [1, LORA_MAX_SLICES] and a slice without pool before touching the GPU."""
    L = lora.lib()
    info = lora.PlanInfo()
    arr = (lora.SliceDesc * 5)()
    assert L.lora_linear_multi(None, 1, 1, 1, 1, 1, ctypes.byref(info), 1, 0, None) == lora.LORA_EINVAL
    for n in (0, -1, lora.LORA_MAX_SLICES + 1):
        assert L.lora_linear_multi(arr, n, 1, 1, 1, 1, ctypes.byref(info), 1, 0, None) == lora.LORA_EINVAL
    assert L.lora_linear_multi(arr, 1, 1, 1, 1, 1, ctypes.byref(info), 1, 0, None) == lora.LORA_EINVAL
    assert L.lora_workspace_bytes_multi(None, 1, 10) == 0
    assert L.lora_workspace_bytes_multi(arr, 2, 10) == 0
    with pytest.raises(ValueError):
        lora.linear_multi(None, [], [], None)


def test_device_plan_sizes_and_argument_errors():
    """Sizes of the device plan buffer, and the host-side refusals of the
    device planner and of lora_linear_device_plan (no kernel launched)."""
    L = lora.lib()
    # T = 64, S = 9: capacity 64 / 16 + 8 = 12 items -> 4 * 12 + 64 + 10 + 8 words
    assert L.lora_plan_device_words(64, 9) == 4 * 12 + 64 + 10 + 8
    assert L.lora_plan_device_words(0, 5) == 4 * 1 + 0 + 6 + 8
    assert L.lora_plan_device_words(10, 0) == 0
    assert L.lora_plan_device_words(-1, 5) == 0
    assert L.lora_plan_device_words(10, lora.LORA_DEVICE_PLAN_MAX_SLOTS + 1) == 0
    assert L.lora_plan_device(0, 1, 10, 1, None) == lora.LORA_EINVAL
    assert L.lora_plan_device(5, 1, 10, None, None) == lora.LORA_EINVAL
    assert L.lora_plan_device(5, None, 10, 1, None) == lora.LORA_EINVAL
    assert L.lora_plan_device(5, 1, -1, 1, None) == lora.LORA_EINVAL
    assert L.lora_plan_device(lora.LORA_DEVICE_PLAN_MAX_SLOTS + 1, 1, 10, 1, None) == lora.LORA_EINVAL
    assert L.lora_linear_device_plan(None, 1, 1, 1, 10, 1, 1, 1 << 20, None) == lora.LORA_EINVAL


def test_bgmv_shrink_argument_errors():
    L = lora.lib()
    assert L.lora_shrink_bgmv(None, 1, 1, 4, 1, 1, 1 << 20, None) == lora.LORA_EINVAL


def test_delta_argument_errors():
    L = lora.lib()
    info = lora.PlanInfo()
    assert L.lora_delta(None, 1, 1, 1, 1, ctypes.byref(info), 1, 1, 1 << 20, None) == lora.LORA_EINVAL
    assert L.lora_delta_bgmv(None, 1, 1, 4, 1, 1, 1 << 20, None) == lora.LORA_EINVAL
