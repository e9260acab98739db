"""Python binding of liblora (include/lora.h): argument marshalling only.

Every step of the layer runs in the library: the planner in its host C++,
the GEMM, shrink, expand and pool writes in its gfx950 kernels. PyTorch is
used for device memory and streams (``torch.cuda.current_stream()``); the
library must be built (``python -m rank_gemm_amd.build``) and there is no
fallback of any kind: if it is missing, or no GPU is present, calls raise.

Names follow the C ABI: ``Pool.install`` -> lora_pool_install, ``plan`` ->
lora_plan, ``linear`` -> lora_linear, ``shrink`` -> lora_shrink.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblora.so")

LORA_OK, LORA_EINVAL, LORA_ESLOT, LORA_ERANK, LORA_ENONFINITE, LORA_EHIP, LORA_ESPACE = 0, -1, -2, -3, -4, -5, -6
LORA_F32, LORA_BF16 = 0, 1
LORA_PLAN_ROWS = 16

EXPORTS = (
    "lora_pool_create", "lora_pool_destroy", "lora_pool_install", "lora_pool_clear", "lora_pool_rank",
    "lora_plan", "lora_plan_max_items", "lora_workspace_bytes", "lora_linear", "lora_shrink",
    "lora_status_string", "lora_profile_begin", "lora_profile_end", "lora_workspace_bytes_multi",
    "lora_linear_multi", "lora_plan_device_words", "lora_plan_device", "lora_linear_device_plan",
    "lora_shrink_bgmv", "lora_linear_multi_device_plan", "lora_plan_chunked", "lora_delta", "lora_delta_bgmv",
    "lora_linear_noalloc", "lora_plan_upload",
)
LORA_DEVICE_PLAN_MAX_SLOTS = 4096
LORA_NOALLOC_MAX_WORKSPACE = 32 << 20
LORA_MAX_SLICES = 4

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_CODE = {"bf16": LORA_BF16, "f32": LORA_F32}


class LoraError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class PlanInfo(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("S", ctypes.c_int32), ("T_a", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n_items", ctypes.c_int32), ("max_seg", ctypes.c_int32), ("chunk", ctypes.c_int32)]


class SliceDesc(ctypes.Structure):
    """lora_slice: one projection of a multi-slice call."""
    _fields_ = [("pool", ctypes.c_void_p), ("W", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("count", ctypes.c_int32), ("mean_ms", ctypes.c_double),
                ("min_ms", ctypes.c_double), ("max_ms", ctypes.c_double), ("median_ms", ctypes.c_double)]


_lib = None
_lock = threading.Lock()
_P, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def lib():
    """Load liblora.so (raises if it was not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_gemm_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            L.lora_pool_create.argtypes = [ctypes.POINTER(_P), _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
            L.lora_pool_destroy.argtypes = [_P]
            L.lora_pool_destroy.restype = None
            L.lora_pool_install.argtypes = [_P, _I, _P, _P, _I, _F, _P]
            L.lora_pool_clear.argtypes = [_P, _I, _P]
            L.lora_pool_rank.argtypes = [_P, _I]
            L.lora_plan.argtypes = [_I, _P, _I, _P, _P, _P, _I, ctypes.POINTER(PlanInfo)]
            L.lora_plan_max_items.argtypes = [_I, _I]
            L.lora_plan_chunked.argtypes = [_I, _P, _I, _I, _P, _P, _P, _I, ctypes.POINTER(PlanInfo)]
            L.lora_delta.argtypes = [_P, _P, _P, _P, _P, ctypes.POINTER(PlanInfo), _P, _P, _SZ, _P]
            L.lora_delta_bgmv.argtypes = [_P, _P, _P, _I, _P, _P, _SZ, _P]
            L.lora_linear_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PlanInfo), _P, _P]
            L.lora_workspace_bytes.argtypes = [_P, _I]
            L.lora_workspace_bytes.restype = _SZ
            L.lora_linear.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PlanInfo), _P, _P, _SZ, _P]
            L.lora_workspace_bytes_multi.argtypes = [ctypes.POINTER(SliceDesc), _I, _I]
            L.lora_workspace_bytes_multi.restype = _SZ
            L.lora_linear_multi.argtypes = [ctypes.POINTER(SliceDesc), _I, _P, _P, _P, _P, ctypes.POINTER(PlanInfo),
                                            _P, _SZ, _P]
            L.lora_plan_device_words.argtypes = [_I, _I]
            L.lora_plan_device_words.restype = _SZ
            L.lora_plan_device.argtypes = [_I, _P, _I, _P, _P]
            L.lora_plan_upload.argtypes = [_P, _P, _SZ, _P]
            L.lora_linear_device_plan.argtypes = [_P, _P, _P, _P, _I, _P, _P, _SZ, _P]
            L.lora_linear_multi_device_plan.argtypes = [ctypes.POINTER(SliceDesc), _I, _P, _P, _I, _P, _SZ, _P]
            L.lora_shrink_bgmv.argtypes = [_P, _P, _P, _I, _P, _P, _SZ, _P]
            L.lora_shrink.argtypes = [_P, _P, _P, _P, _P, ctypes.POINTER(PlanInfo), _P, _P, _SZ, _P]
            L.lora_profile_begin.argtypes = [_I]
            L.lora_profile_end.argtypes = [ctypes.POINTER(KernelStat), _I, ctypes.POINTER(_I)]
            L.lora_status_string.argtypes = [_I]
            L.lora_status_string.restype = ctypes.c_char_p
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lora_status_string(int(status)).decode()


def _check(rc: int, what: str):
    if rc != LORA_OK:
        raise LoraError(rc, what)


def _require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("liblora needs a HIP GPU; none is visible")


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev_tensor(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host array from rank_gemm_amd.inputs (uint16 bf16 bits or float32) ->
    device tensor of the pool's element type (bits unchanged)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, np.float32))
    return t.to(device)


class Pool:
    """Device slot pool: A [S, r_max, d_in], B [S, d_out, r_max], rank [S],
    scale [S]; slot 0 is the zero adapter."""

    def __init__(self, S: int, r_max: int, d_in: int, d_out: int, dtype: str = "bf16", device="cuda"):
        _require_gpu()
        self.S, self.r_max, self.d_in, self.d_out, self.dtype = S, r_max, d_in, d_out, dtype
        self.device = torch.device(device)
        tdt = _TORCH_DTYPE[dtype]
        with torch.cuda.device(self.device):
            self.A = torch.empty((S, r_max, d_in), dtype=tdt, device=self.device)
            self.B = torch.empty((S, d_out, r_max), dtype=tdt, device=self.device)
            self.rank_dev = torch.empty(S, dtype=torch.int32, device=self.device)
            self.scale_dev = torch.empty(S, dtype=torch.float32, device=self.device)
            h = _P()
            _check(lib().lora_pool_create(ctypes.byref(h), S, r_max, d_in, d_out, _CODE[dtype], self.A.data_ptr(),
                                          self.B.data_ptr(), self.rank_dev.data_ptr(), self.scale_dev.data_ptr(),
                                          _stream(self.device)), "lora_pool_create")
        self._h = h
        self._ws = {}  # stream handle -> workspace
        self._ws_retired = []

    @property
    def handle(self):
        return self._h

    def install(self, slot: int, A: torch.Tensor, B: torch.Tensor, alpha: float):
        """lora_pool_install: A [r, d_in], B [d_out, r] device tensors."""
        tdt = _TORCH_DTYPE[self.dtype]
        if A.dim() != 2 or B.dim() != 2:
            raise ValueError("A and B must be 2-D")
        r = A.shape[0]
        _dev_tensor(A, tdt, "A", (r, self.d_in))
        _dev_tensor(B, tdt, "B", (self.d_out, r))
        with torch.cuda.device(self.device):
            _check(lib().lora_pool_install(self._h, int(slot), A.data_ptr(), B.data_ptr(), int(r), float(alpha),
                                           _stream(self.device)), "lora_pool_install")

    def clear(self, slot: int):
        with torch.cuda.device(self.device):
            _check(lib().lora_pool_clear(self._h, int(slot), _stream(self.device)), "lora_pool_clear")

    def rank(self, slot: int) -> int:
        return lib().lora_pool_rank(self._h, int(slot))

    def workspace_bytes(self, T: int) -> int:
        return int(lib().lora_workspace_bytes(self._h, int(T)))

    def workspace(self, T: int) -> torch.Tensor:
        """A device workspace of at least workspace_bytes(T) for calls on the
        current stream. One buffer per stream, so calls on two streams never
        share one; calls on one stream reuse it in stream order. A buffer
        that grows is replaced, but the old one is kept until the pool is
        released (a captured graph or a call still in flight may use it)."""
        n = self.workspace_bytes(T)
        key = torch.cuda.current_stream(self.device).cuda_stream
        ws = self._ws.get(key)
        if ws is None or ws.numel() < n:
            if ws is not None:
                self._ws_retired.append(ws)
            ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.lora_pool_destroy(h)
            self._h = None


class Plan:
    """Host result of lora_plan plus its device copy."""

    def __init__(self, S, T, info, host, dev, n_work, chunk=LORA_PLAN_ROWS):
        self.S, self.T, self.info, self.chunk = S, T, info, chunk
        self.host = host  # pinned int32: [work 4*n_work][token_order T][slot_indptr S+1]
        self.dev = dev
        self._n_work = n_work
        # plan_into staging: two pinned buffers used in turn, the copy that
        # last read each (None: not read yet), the one to write next
        self._stage, self._ev, self._turn = [None, None], [None, None], 0

    def _off(self, which):
        if which == "work":
            return 0
        if which == "token_order":
            return 4 * self._n_work
        return 4 * self._n_work + self.T

    @property
    def token_order(self) -> np.ndarray:
        o = self._off("token_order")
        return self.host[o:o + self.T].numpy()

    @property
    def slot_indptr(self) -> np.ndarray:
        o = self._off("slot_indptr")
        return self.host[o:o + self.S + 1].numpy()

    @property
    def work(self) -> np.ndarray:
        return self.host[: 4 * self.info.n_items].numpy().reshape(-1, 4)

    def dev_ptrs(self):
        base = self.dev.data_ptr() if self.dev is not None else 0
        return (base + 4 * self._off("token_order"), base + 4 * self._off("slot_indptr"), base + 4 * self._off("work"))


def plan(slot_ids, S: int, device="cuda", upload: bool = True, chunk: int = LORA_PLAN_ROWS) -> Plan:
    """lora_plan (or lora_plan_chunked for ``chunk`` of 32, 64 or 128 rows
    per work item) over host slot ids; with ``upload`` the result is copied
    to ``device`` on the current stream (non-blocking, from pinned memory).
    lora_linear, lora_linear_multi and lora_shrink take 16-row plans only;
    lora_delta takes any chunk."""
    ids = np.ascontiguousarray(np.asarray(slot_ids), dtype=np.int32)
    if ids.ndim != 1:
        raise ValueError("slot_ids must be 1-D")
    T = int(ids.shape[0])
    n_work = max(int(lib().lora_plan_max_items(T, int(S))), 1)
    total = 4 * n_work + T + S + 1
    pin = upload and torch.cuda.is_available()
    host = torch.empty(total, dtype=torch.int32, pin_memory=pin)
    base = host.data_ptr()
    info = PlanInfo()
    _check(lib().lora_plan_chunked(int(S), ids.ctypes.data, T, int(chunk), base + 16 * n_work,
                                   base + 4 * (4 * n_work + T), base, n_work, ctypes.byref(info)),
           "lora_plan_chunked")
    dev = None
    if upload:
        _require_gpu()
        dev = torch.empty(total, dtype=torch.int32, device=device)
        with torch.cuda.device(dev.device):
            _check(lib().lora_plan_upload(base, dev.data_ptr(), total, _stream(dev.device)), "lora_plan_upload")
    p = Plan(int(S), T, info, host, dev, n_work, int(chunk))
    if upload:
        # the staging buffers of plan_into, allocated now rather than on
        # first use: pinning host memory stalls the kernels running then
        ev = torch.cuda.Event()
        ev.record()
        p._stage = [host, torch.empty(total, dtype=torch.int32, pin_memory=True)]
        p._ev = [ev, None]
        p._turn = 1
    return p


def plan_into(p: Plan, slot_ids) -> Plan:
    """Re-plan ``slot_ids`` into the device buffer of an existing plan (same
    T and S, same chunk), so work captured against that buffer sees the new
    plan. The summary (p.info) is refreshed; kernels captured with an older
    summary stay valid only while it is unchanged, which the caller checks.

    The plan is written into one of two pinned staging buffers that the plan
    owns for its lifetime (the first is the buffer lora_plan filled), in
    turn, and copied from there on the current stream by lora_plan_upload
    (a kernel reading the pinned buffer in place). Before a staging
    buffer is written again, the host waits for the copy that last read it
    (two plans back). No pinned memory is allocated here: registering new
    host memory with the GPU stalls the kernels running at that moment."""
    ids = np.ascontiguousarray(np.asarray(slot_ids), dtype=np.int32)
    if ids.ndim != 1 or ids.shape[0] != p.T:
        raise ValueError("plan_into needs the same T and S")
    if p.dev is None:
        raise ValueError("plan was not uploaded")
    k = p._turn
    p._turn ^= 1
    if p._ev[k] is None:
        p._ev[k] = torch.cuda.Event()
    else:
        p._ev[k].synchronize()
    host = p._stage[k]
    base = host.data_ptr()
    info = PlanInfo()
    _check(lib().lora_plan_chunked(int(p.S), ids.ctypes.data, p.T, p.chunk, base + 16 * p._n_work,
                                   base + 4 * (4 * p._n_work + p.T), base, p._n_work, ctypes.byref(info)),
           "lora_plan_chunked")
    with torch.cuda.device(p.dev.device):
        _check(lib().lora_plan_upload(base, p.dev.data_ptr(), int(p.dev.numel()), _stream(p.dev.device)),
               "lora_plan_upload")
    p._ev[k].record()
    p.host, p.info = host, info
    return p


class DevicePlan:
    """A plan built on the device by lora_plan_device: one int32 buffer
    [work 4 W][token_order T][slot_indptr S + 1][info 8]."""

    def __init__(self, S: int, T: int, buf: torch.Tensor):
        self.S, self.T, self.buf = S, T, buf
        self.cap = max(int(lib().lora_plan_max_items(T, S)), 1)

    def read(self) -> dict:
        """Copy the plan to the host (synchronises): work (live items only),
        token_order, slot_indptr and the info words."""
        h = self.buf.cpu().numpy()
        o = 4 * self.cap
        info = h[o + self.T + self.S + 1:]
        keys = ("T", "S", "T_a", "k", "n_items", "max_seg", "status")
        d = {k: int(v) for k, v in zip(keys, info)}
        d["work"] = h[:4 * d["n_items"]].reshape(-1, 4)
        d["pad"] = h[4 * d["n_items"]:o].reshape(-1, 4)
        d["token_order"] = h[o:o + self.T]
        d["slot_indptr"] = h[o + self.T:o + self.T + self.S + 1]
        return d


def plan_device(slot_ids: torch.Tensor, S: int, out: DevicePlan | None = None) -> DevicePlan:
    """lora_plan_device: plan device-resident int32 slot ids on the current
    stream (no host work; graph-capturable). ``out`` reuses a buffer of the
    same T and S."""
    _dev_tensor(slot_ids, torch.int32, "slot_ids")
    if slot_ids.dim() != 1:
        raise ValueError("slot_ids must be 1-D")
    T = int(slot_ids.shape[0])
    words = int(lib().lora_plan_device_words(T, int(S)))
    if words == 0:
        raise ValueError(f"no device plan for T={T}, S={S} (1 <= S <= {LORA_DEVICE_PLAN_MAX_SLOTS})")
    if out is None:
        out = DevicePlan(int(S), T, torch.empty(words, dtype=torch.int32, device=slot_ids.device))
    elif out.T != T or out.S != S:
        raise ValueError("plan buffer has another T or S")
    _check(lib().lora_plan_device(int(S), slot_ids.data_ptr(), T, out.buf.data_ptr(), _stream(slot_ids.device)),
           "lora_plan_device")
    return out


def linear(x: torch.Tensor, W: torch.Tensor, pool: Pool, p, y: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """lora_linear (host plan) or lora_linear_device_plan (DevicePlan):
    y = x W^T + per-row adapter correction."""
    tdt = _TORCH_DTYPE[pool.dtype]
    T = p.T
    _dev_tensor(x, tdt, "x", (T, pool.d_in))
    _dev_tensor(W, tdt, "W", (pool.d_out, pool.d_in))
    if y is None:
        y = torch.empty((T, pool.d_out), dtype=tdt, device=x.device)
    _dev_tensor(y, tdt, "y", (T, pool.d_out))
    ws = workspace if workspace is not None else pool.workspace(T)
    if isinstance(p, DevicePlan):
        if p.S != pool.S:
            raise ValueError("plan and pool have different S")
        _check(lib().lora_linear_device_plan(pool.handle, x.data_ptr(), W.data_ptr(), p.buf.data_ptr(), T,
                                             y.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                             _stream(x.device)), "lora_linear_device_plan")
        return y
    if p.dev is None:
        raise ValueError("plan was not uploaded")
    to, ip, wk = p.dev_ptrs()
    _check(lib().lora_linear(pool.handle, x.data_ptr(), W.data_ptr(), to, ip, wk, ctypes.byref(p.info), y.data_ptr(),
                             ws.data_ptr(), ws.numel() * ws.element_size(), _stream(x.device)), "lora_linear")
    return y


def _slice_array(pools, Ws=None, ys=None):
    n = len(pools)
    arr = (SliceDesc * max(n, 1))()
    for i, pool in enumerate(pools):
        arr[i].pool = pool.handle
        arr[i].W = Ws[i].data_ptr() if Ws is not None else None
        arr[i].y = ys[i].data_ptr() if ys is not None else None
    return arr


def workspace_bytes_multi(pools, T: int) -> int:
    """lora_workspace_bytes_multi (0 when the pools cannot share a call)."""
    return int(lib().lora_workspace_bytes_multi(_slice_array(pools, None, None), len(pools), int(T)))


def linear_multi(x: torch.Tensor, Ws, pools, p: Plan, ys=None, workspace: torch.Tensor | None = None):
    """lora_linear_multi: y_i = x W_i^T + per-row correction from pools[i],
    for slices that share x and the plan (a merged q/k/v or gate/up)."""
    n = len(pools)
    if not 1 <= n <= LORA_MAX_SLICES or len(Ws) != n:
        raise ValueError(f"need 1..{LORA_MAX_SLICES} pools and as many weights")
    tdt = _TORCH_DTYPE[pools[0].dtype]
    T = p.T
    _dev_tensor(x, tdt, "x", (T, pools[0].d_in))
    if not isinstance(p, DevicePlan) and p.dev is None:
        raise ValueError("plan was not uploaded")
    if ys is None:
        ys = [torch.empty((T, pl.d_out), dtype=tdt, device=x.device) for pl in pools]
    for i, pl in enumerate(pools):
        _dev_tensor(Ws[i], tdt, f"W[{i}]", (pl.d_out, pl.d_in))
        _dev_tensor(ys[i], tdt, f"y[{i}]", (T, pl.d_out))
    arr = _slice_array(pools, Ws, ys)
    if workspace is None:
        need = int(lib().lora_workspace_bytes_multi(arr, n, T))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if isinstance(p, DevicePlan):
        if p.S != pools[0].S:
            raise ValueError("plan and pools have different S")
        _check(lib().lora_linear_multi_device_plan(arr, n, x.data_ptr(), p.buf.data_ptr(), T, workspace.data_ptr(),
                                                   workspace.numel() * workspace.element_size(), _stream(x.device)),
               "lora_linear_multi_device_plan")
        return ys
    to, ip, wk = p.dev_ptrs()
    _check(lib().lora_linear_multi(arr, n, x.data_ptr(), to, ip, wk, ctypes.byref(p.info), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream(x.device)),
           "lora_linear_multi")
    return ys


def shrink(x: torch.Tensor, pool: Pool, p: Plan, h: torch.Tensor | None = None) -> torch.Tensor:
    """lora_shrink: h [T, r_max] fp32 (zeros past each row's rank)."""
    tdt = _TORCH_DTYPE[pool.dtype]
    _dev_tensor(x, tdt, "x", (p.T, pool.d_in))
    if h is None:
        h = torch.empty((p.T, pool.r_max), dtype=torch.float32, device=x.device)
    _dev_tensor(h, torch.float32, "h", (p.T, pool.r_max))
    ws = pool.workspace(p.T)
    to, ip, wk = p.dev_ptrs()
    _check(lib().lora_shrink(pool.handle, x.data_ptr(), to, ip, wk, ctypes.byref(p.info), h.data_ptr(), ws.data_ptr(),
                             ws.numel(), _stream(x.device)), "lora_shrink")
    return h


def shrink_bgmv(x: torch.Tensor, pool: Pool, slot_ids: torch.Tensor, h: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """lora_shrink_bgmv: h [T, r_max] fp32 in token order from device slot ids (no plan)."""
    tdt = _TORCH_DTYPE[pool.dtype]
    _dev_tensor(slot_ids, torch.int32, "slot_ids")
    T = int(slot_ids.shape[0])
    _dev_tensor(x, tdt, "x", (T, pool.d_in))
    if h is None:
        h = torch.empty((T, pool.r_max), dtype=torch.float32, device=x.device)
    _dev_tensor(h, torch.float32, "h", (T, pool.r_max))
    ws = workspace if workspace is not None else pool.workspace(T)
    _check(lib().lora_shrink_bgmv(pool.handle, x.data_ptr(), slot_ids.data_ptr(), T, h.data_ptr(), ws.data_ptr(),
                                  ws.numel() * ws.element_size(), _stream(x.device)), "lora_shrink_bgmv")
    return h


def correction(x: torch.Tensor, pool: Pool, p: Plan, y: torch.Tensor,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """lora_delta: y += per-row adapter correction (SGMV over a plan of any
    chunk); rows on slot 0 are not touched."""
    tdt = _TORCH_DTYPE[pool.dtype]
    _dev_tensor(x, tdt, "x", (p.T, pool.d_in))
    _dev_tensor(y, tdt, "y", (p.T, pool.d_out))
    if p.dev is None:
        raise ValueError("plan was not uploaded")
    ws = workspace if workspace is not None else pool.workspace(p.T)
    to, ip, wk = p.dev_ptrs()
    _check(lib().lora_delta(pool.handle, x.data_ptr(), to, ip, wk, ctypes.byref(p.info), y.data_ptr(), ws.data_ptr(),
                            ws.numel() * ws.element_size(), _stream(x.device)), "lora_delta")
    return y


def correction_bgmv(x: torch.Tensor, pool: Pool, slot_ids: torch.Tensor, y: torch.Tensor,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """lora_delta_bgmv: y += per-row adapter correction, token by token from
    device slot ids (no plan)."""
    tdt = _TORCH_DTYPE[pool.dtype]
    _dev_tensor(slot_ids, torch.int32, "slot_ids")
    T = int(slot_ids.shape[0])
    _dev_tensor(x, tdt, "x", (T, pool.d_in))
    _dev_tensor(y, tdt, "y", (T, pool.d_out))
    ws = workspace if workspace is not None else pool.workspace(T)
    _check(lib().lora_delta_bgmv(pool.handle, x.data_ptr(), slot_ids.data_ptr(), T, y.data_ptr(), ws.data_ptr(),
                                 ws.numel() * ws.element_size(), _stream(x.device)), "lora_delta_bgmv")
    return y


def profile_begin(max_records: int = 100000):
    """lora_profile_begin: start recording per-kernel HIP event pairs."""
    _check(lib().lora_profile_begin(int(max_records)), "lora_profile_begin")


def profile_end() -> dict:
    """lora_profile_end: {kernel name: {count, mean_ms, min_ms, max_ms, median_ms}}."""
    cap = 32
    out = (KernelStat * cap)()
    n = _I()
    _check(lib().lora_profile_end(out, cap, ctypes.byref(n)), "lora_profile_end")
    return {out[i].name.decode(): {"count": out[i].count, "mean_ms": out[i].mean_ms, "min_ms": out[i].min_ms,
                                   "max_ms": out[i].max_ms, "median_ms": out[i].median_ms}
            for i in range(min(n.value, cap))}
