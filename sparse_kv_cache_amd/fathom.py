"""Thin Python binding of libfathom (ctypes).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and streams.  The library must have
been built (``python -m sparse_kv_cache_amd.build``); importing this module
raises if it is missing -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfathom.so")

FATHOM_OK = 0
FATHOM_ERR_INVALID_ARG = -1
FATHOM_ERR_UNSUPPORTED = -2
FATHOM_ERR_WORKSPACE = -3
FATHOM_ERR_HIP = -4
FATHOM_OP_PACK = 0
FATHOM_OP_SCAN = 1
FATHOM_OP_ATTEND = 2
FATHOM_CONTROL_UNIFORM = 0
FATHOM_CONTROL_TOP_CHANNELS = 1
FATHOM_STAGE_COPY_ENGINE = 0
FATHOM_STAGE_GATHER = 1
MAX_K = 4096
NOALLOC_MAX_Q = 64
NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "fathom_plane_ldw",
    "fathom_workspace_bytes",
    "fathom_pack_planes",
    "fathom_append_keys",
    "fathom_allocate",
    "fathom_control_allocate",
    "fathom_scan_topk",
    "fathom_allocate_scan_topk",
    "fathom_allocate_scan_topk_noalloc",
    "fathom_allocate_scan_topk_staged",
    "fathom_sparse_attention",
    "fathom_host_device_pointer",
    "fathom_status_string",
    "fathom_last_error",
    "fathom_timing_enable",
    "fathom_timing_read",
    "fathom_stream_read",
    "fathom_stream_read_sink_words",
)


class StoreDesc(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("n", ctypes.c_int64),
        ("ldw", ctypes.c_int64),
        ("lengths", ctypes.c_void_p),
    ]


class FathomError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {detail}")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} not found: build it with `python -m sparse_kv_cache_amd.build` "
            "(the Fathom path has no CPU fallback)"
        )
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SD = ctypes.POINTER(StoreDesc)
    sig = {
        "fathom_plane_ldw": (i64, [i64]),
        "fathom_workspace_bytes": (sz, [i32, SD, i32, i32]),
        "fathom_pack_planes": (ctypes.c_int, [P, i64, i64, SD, P, P, P, P, P, sz, P]),
        "fathom_append_keys": (ctypes.c_int, [P, i64, i64, i32, SD, P, P, P, P]),
        "fathom_allocate": (ctypes.c_int, [P, i32, i32, P, SD, i32, P, P]),
        "fathom_control_allocate": (ctypes.c_int, [P, i32, i32, i32, P, P]),
        "fathom_scan_topk": (ctypes.c_int, [P, P, P, SD, P, P, i32, i32, i32, P, P, P, P, sz, P]),
        "fathom_allocate_scan_topk": (ctypes.c_int, [P, P, P, P, SD, P, i32, i32, i32, i32, P, P, P, P, sz, P]),
        "fathom_allocate_scan_topk_noalloc": (ctypes.c_int, [P, P, P, P, SD, P, i32, i32, i32, i32, P, P, P, P]),
        "fathom_allocate_scan_topk_staged": (ctypes.c_int, [P, P, P, P, SD, P, i32, i32, i32, i32, P, P, P, P, sz, P,
                                                            sz, i32, P, P]),
        "fathom_sparse_attention": (ctypes.c_int, [P, P, i64, i64, SD, P, P, i32, i32, i32, ctypes.c_float, P, P,
                                                   sz, P]),
        "fathom_host_device_pointer": (ctypes.c_int, [P, ctypes.POINTER(P)]),
        "fathom_status_string": (ctypes.c_char_p, [i32]),
        "fathom_last_error": (ctypes.c_char_p, []),
        "fathom_timing_enable": (ctypes.c_int, [i32]),
        "fathom_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]),
        "fathom_stream_read": (ctypes.c_int, [P, i64, P, P]),
        "fathom_stream_read_sink_words": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int, where: str):
    if status != FATHOM_OK:
        raise FathomError(status, where, lib.fathom_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def plane_ldw(n: int) -> int:
    return int(lib.fathom_plane_ldw(n))


def store_desc(num_kv_heads: int, n: int, d: int = 128, ldw: Optional[int] = None,
               lengths: Optional[torch.Tensor] = None) -> StoreDesc:
    """Store descriptor; ``lengths`` (int32 [H] on the GPU) gives each head its
    own number of keys (at most n).  The caller keeps that tensor alive."""
    if lengths is not None:
        assert lengths.dtype == torch.int32 and lengths.numel() == num_kv_heads and lengths.is_contiguous()
    return StoreDesc(num_kv_heads, d, n, plane_ldw(n) if ldw is None else ldw,
                     None if lengths is None else lengths.data_ptr())


def workspace_bytes(op: int, store: StoreDesc, num_q: int = 1, k: int = 1) -> int:
    return int(lib.fathom_workspace_bytes(op, ctypes.byref(store), num_q, k))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns >= 512-byte aligned blocks
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def pack_planes(keys: torch.Tensor, store: Optional[StoreDesc] = None, *, with_var: bool = True,
                planes: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None):
    """keys: float32 [H, n, d] on the GPU (token stride may exceed d).
    Returns (planes uint32 [H, d, 4, ldw] viewed as int32, lo, step, var)."""
    assert keys.dtype == torch.float32 and keys.dim() == 3 and keys.stride(2) == 1
    H, n, d = keys.shape
    store = store or store_desc(H, n, d)
    dev = keys.device
    if planes is None:
        planes = torch.empty((H, d, 4, store.ldw), dtype=torch.int32, device=dev)
    lo = torch.empty((H, d), dtype=torch.float32, device=dev)
    step = torch.empty((H, d), dtype=torch.float32, device=dev)
    var = torch.empty((H, d), dtype=torch.float32, device=dev) if with_var else None
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(FATHOM_OP_PACK, store), dev)
    st = lib.fathom_pack_planes(_ptr(keys), keys.stride(0), keys.stride(1), ctypes.byref(store),
                                _ptr(planes), _ptr(lo), _ptr(step), _ptr(var), _ptr(workspace),
                                workspace.numel(), _stream(stream))
    _check(st, "fathom_pack_planes")
    return planes, lo, step, var


def append_keys(keys: torch.Tensor, store: StoreDesc, planes: torch.Tensor, lo: torch.Tensor,
                step: torch.Tensor, stream=None) -> StoreDesc:
    """Write keys float32 [H, m, d] (token stride may exceed d) as keys
    store.n .. store.n + m - 1 of every head (with per-head lengths: at each
    head's own length, which grows by m); returns the store grown by m."""
    assert keys.dtype == torch.float32 and keys.dim() == 3 and keys.stride(2) == 1
    H, m, d = keys.shape
    st = lib.fathom_append_keys(_ptr(keys), keys.stride(0), keys.stride(1), m, ctypes.byref(store), _ptr(planes),
                                _ptr(lo), _ptr(step), _stream(stream))
    _check(st, "fathom_append_keys")
    return StoreDesc(store.num_kv_heads, store.d, store.n + m, store.ldw, store.lengths)


def allocate(q: torch.Tensor, var: torch.Tensor, group: int, budget: int,
             store: Optional[StoreDesc] = None, out: Optional[torch.Tensor] = None, stream=None):
    """q float32 [Q, d], var float32 [H, d] -> alloc uint8 [Q, d]."""
    Q, d = q.shape
    H = var.shape[0]
    store = store or StoreDesc(H, d, 1, 4)
    if out is None:
        out = torch.empty((Q, d), dtype=torch.uint8, device=q.device)
    st = lib.fathom_allocate(_ptr(q), Q, group, _ptr(var), ctypes.byref(store), budget, _ptr(out),
                             _stream(stream))
    _check(st, "fathom_allocate")
    return out


def control_allocate(q: torch.Tensor, mode: int, budget: int, out: Optional[torch.Tensor] = None, stream=None):
    """Fixed-depth control allocation (FATHOM_CONTROL_*): q float32 [Q, d] -> uint8 [Q, d]."""
    Q, d = q.shape
    if out is None:
        out = torch.empty((Q, d), dtype=torch.uint8, device=q.device)
    st = lib.fathom_control_allocate(_ptr(q), Q, mode, budget, _ptr(out), _stream(stream))
    _check(st, "fathom_control_allocate")
    return out


def scan_topk(planes: torch.Tensor, lo: torch.Tensor, step: torch.Tensor, store: StoreDesc,
              q: torch.Tensor, alloc: torch.Tensor, group: int, k: int, *,
              all_scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              out_idx: Optional[torch.Tensor] = None, out_score: Optional[torch.Tensor] = None,
              planes_ptr: Optional[int] = None, stream=None):
    """Top-k keys per query: (idx int32 [Q, k], score float32 [Q, k]).

    ``planes_ptr`` overrides the plane store address (for a store in pinned
    host memory, pass its device-visible address)."""
    Q = q.shape[0]
    dev = q.device
    if out_idx is None:
        out_idx = torch.empty((Q, k), dtype=torch.int32, device=dev)
    if out_score is None:
        out_score = torch.empty((Q, k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(FATHOM_OP_SCAN, store, Q, k), dev)
    pp = ctypes.c_void_p(planes_ptr) if planes_ptr is not None else _ptr(planes)
    st = lib.fathom_scan_topk(pp, _ptr(lo), _ptr(step), ctypes.byref(store), _ptr(q), _ptr(alloc),
                              Q, group, k, _ptr(out_idx), _ptr(out_score), _ptr(all_scores),
                              _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "fathom_scan_topk")
    return out_idx, out_score


def allocate_scan_topk(planes: torch.Tensor, lo: torch.Tensor, step: torch.Tensor, var: torch.Tensor,
                       store: StoreDesc, q: torch.Tensor, group: int, budget: int, k: int, *,
                       workspace: Optional[torch.Tensor] = None, alloc: Optional[torch.Tensor] = None,
                       out_idx: Optional[torch.Tensor] = None, out_score: Optional[torch.Tensor] = None,
                       planes_ptr: Optional[int] = None, stream=None):
    """allocate() then scan_topk() in one call: (alloc uint8 [Q, d], idx, score)."""
    Q, d = q.shape
    dev = q.device
    if alloc is None:
        alloc = torch.empty((Q, d), dtype=torch.uint8, device=dev)
    if out_idx is None:
        out_idx = torch.empty((Q, k), dtype=torch.int32, device=dev)
    if out_score is None:
        out_score = torch.empty((Q, k), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(FATHOM_OP_SCAN, store, Q, k), dev)
    pp = ctypes.c_void_p(planes_ptr) if planes_ptr is not None else _ptr(planes)
    st = lib.fathom_allocate_scan_topk(pp, _ptr(lo), _ptr(step), _ptr(var), ctypes.byref(store), _ptr(q),
                                       Q, group, budget, k, _ptr(alloc), _ptr(out_idx), _ptr(out_score),
                                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "fathom_allocate_scan_topk")
    return alloc, out_idx, out_score


def allocate_scan_topk_noalloc(planes: torch.Tensor, lo: torch.Tensor, step: torch.Tensor, var: torch.Tensor,
                               store: StoreDesc, q: torch.Tensor, group: int, budget: int, k: int, *,
                               alloc: torch.Tensor, out_idx: torch.Tensor, out_score: torch.Tensor,
                               planes_ptr: Optional[int] = None, stream=None):
    """allocate_scan_topk() with the library's static scratch memory: no
    workspace, and nothing allocated here either (every output is passed in)."""
    Q = q.shape[0]
    pp = ctypes.c_void_p(planes_ptr) if planes_ptr is not None else _ptr(planes)
    st = lib.fathom_allocate_scan_topk_noalloc(pp, _ptr(lo), _ptr(step), _ptr(var), ctypes.byref(store), _ptr(q),
                                               Q, group, budget, k, _ptr(alloc), _ptr(out_idx), _ptr(out_score),
                                               _stream(stream))
    _check(st, "fathom_allocate_scan_topk_noalloc")
    return alloc, out_idx, out_score


def staging_bytes(store: StoreDesc) -> int:
    """Device staging the host-resident staged call needs: two head blocks."""
    return 2 * store.d * 4 * store.ldw * 4


def allocate_scan_topk_staged(planes_host: torch.Tensor, lo: torch.Tensor, step: torch.Tensor, var: torch.Tensor,
                              store: StoreDesc, q: torch.Tensor, group: int, budget: int, k: int, *,
                              staging: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              alloc: Optional[torch.Tensor] = None, out_idx: Optional[torch.Tensor] = None,
                              out_score: Optional[torch.Tensor] = None, mode: int = FATHOM_STAGE_GATHER,
                              copy_stream=None, stream=None):
    """allocate_scan_topk() over a plane store in pinned host memory, its
    union rows staged into HBM head by head (FATHOM_STAGE_GATHER: by a
    kernel; FATHOM_STAGE_COPY_ENGINE: by hipMemcpyAsync, blocking until the
    allocation reaches the host).  planes_host: pinned CPU tensor."""
    assert planes_host.is_pinned()
    Q, d = q.shape
    dev = q.device
    if alloc is None:
        alloc = torch.empty((Q, d), dtype=torch.uint8, device=dev)
    if out_idx is None:
        out_idx = torch.empty((Q, k), dtype=torch.int32, device=dev)
    if out_score is None:
        out_score = torch.empty((Q, k), dtype=torch.float32, device=dev)
    if staging is None:
        staging = alloc_workspace(staging_bytes(store), dev)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(FATHOM_OP_SCAN, store, group, k), dev)
    if copy_stream is None:
        copy_stream = torch.cuda.Stream(device=dev)
    st = lib.fathom_allocate_scan_topk_staged(
        _ptr(planes_host), _ptr(lo), _ptr(step), _ptr(var), ctypes.byref(store), _ptr(q), Q, group, budget, k,
        _ptr(alloc), _ptr(out_idx), _ptr(out_score), _ptr(staging), staging.numel() * staging.element_size(),
        _ptr(workspace), workspace.numel(), mode, _stream(stream), _stream(copy_stream))
    _check(st, "fathom_allocate_scan_topk_staged")
    return alloc, out_idx, out_score


def sparse_attention(k_rows: torch.Tensor, v_rows: torch.Tensor, store: StoreDesc, q: torch.Tensor,
                     idx: torch.Tensor, group: int, scale: Optional[float] = None, *,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     k_ptr: Optional[int] = None, v_ptr: Optional[int] = None, stream=None):
    """Attention of each query over its selected rows: k_rows, v_rows bfloat16
    [H, n, d] (channel stride 1; k_ptr / v_ptr override the addresses, e.g.
    for rows in pinned host memory), q float32 [Q, d], idx int32 [Q, k] ->
    out float32 [Q, d]."""
    assert k_rows.dtype == torch.bfloat16 and v_rows.dtype == torch.bfloat16
    H = k_rows.shape[0]
    assert k_rows.shape == v_rows.shape and k_rows.stride(2) == 1 and v_rows.stride(2) == 1
    assert k_rows.stride(1) == v_rows.stride(1) and (H == 1 or k_rows.stride(0) == v_rows.stride(0))
    Q, d = q.shape
    k = idx.shape[1]
    dev = q.device
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty((Q, d), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(workspace_bytes(FATHOM_OP_ATTEND, store, Q, k), dev)
    kp = ctypes.c_void_p(k_ptr) if k_ptr is not None else _ptr(k_rows)
    vp = ctypes.c_void_p(v_ptr) if v_ptr is not None else _ptr(v_rows)
    stride_head = k_rows.stride(0) if H > 1 else k_rows.shape[1] * k_rows.stride(1)
    st = lib.fathom_sparse_attention(kp, vp, stride_head, k_rows.stride(1), ctypes.byref(store), _ptr(q),
                                     _ptr(idx), Q, group, k, float(scale), _ptr(out), _ptr(workspace),
                                     workspace.numel(), _stream(stream))
    _check(st, "fathom_sparse_attention")
    return out


def host_device_pointer(pinned: torch.Tensor) -> int:
    dp = ctypes.c_void_p()
    _check(lib.fathom_host_device_pointer(_ptr(pinned), ctypes.byref(dp)), "fathom_host_device_pointer")
    return int(dp.value)


def timing_enable(on: bool = True):
    _check(lib.fathom_timing_enable(1 if on else 0), "fathom_timing_enable")


def timing_read():
    ms = ctypes.c_double()
    cnt = ctypes.c_int32()
    _check(lib.fathom_timing_read(ctypes.byref(ms), ctypes.byref(cnt)), "fathom_timing_read")
    return ms.value, cnt.value


def stream_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Streaming read of the whole of src (a measurement aid: the HBM read
    ceiling).  Returns the sink buffer."""
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.zeros(int(lib.fathom_stream_read_sink_words()), dtype=torch.int32, device=src.device)
    _check(lib.fathom_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "fathom_stream_read")
    return sink
