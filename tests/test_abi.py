"""Host-side checks of the C ABI: the library loads, exports every function
include/fathom.h declares, sizes workspaces, and rejects invalid arguments
on the host before any HIP call (so these run without a GPU; every call
here is built to fail validation and launches nothing)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fathom.h")

fa = pytest.importorskip("sparse_kv_cache_amd.fathom", reason="libfathom.so not built")
lib = fa.lib
SD = fa.StoreDesc
FAKE = ctypes.c_void_p(0x1000)        # 256-aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(fathom_\w+)\s*\(", text, re.M)))


def test_exports_match_header():
    names = declared_functions()
    assert len(names) == len(fa.EXPORTS) and set(names) == set(fa.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {fa._LIB_PATH}").read()
    for name in names:
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_plane_ldw_and_workspace():
    assert fa.plane_ldw(1) == 4 and fa.plane_ldw(129) == 8 and fa.plane_ldw(1 << 20) == 32768
    assert lib.fathom_plane_ldw(0) == -1
    s = fa.store_desc(8, 1 << 20)
    assert fa.workspace_bytes(fa.FATHOM_OP_PACK, s) >= 8 * 128 * 24
    ws = fa.workspace_bytes(fa.FATHOM_OP_SCAN, s, 32, 2048)
    assert ws >= 32 * (16384 * 8 + 8192 * 4)
    assert fa.workspace_bytes(7, s) == 0
    assert fa.workspace_bytes(fa.FATHOM_OP_SCAN, SD(8, 64, 1 << 20, 32768), 32, 2048) == 0


def status_text(st):
    return lib.fathom_status_string(st).decode()


def test_status_strings():
    assert status_text(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert status_text(st) not in ("ok", "unknown status")
    assert status_text(99) == "unknown status"


def _pack(store, keys=FAKE, stride_head=None, stride_token=128, planes=FAKE, ws=FAKE, ws_bytes=1 << 20):
    if stride_head is None:
        stride_head = store.n * 128
    return lib.fathom_pack_planes(keys, stride_head, stride_token, ctypes.byref(store), planes, FAKE,
                                  FAKE, FAKE, ws, ws_bytes, None)


def test_pack_validation():
    good = SD(2, 128, 1000, fa.plane_ldw(1000))
    assert _pack(SD(2, 64, 1000, 32)) == fa.FATHOM_ERR_UNSUPPORTED
    assert _pack(SD(0, 128, 1000, 32)) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(SD(2, 128, 0, 4)) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(SD(2, 128, 1000, 30)) == fa.FATHOM_ERR_INVALID_ARG      # not a multiple of 4
    assert _pack(SD(2, 128, 1000, 28)) == fa.FATHOM_ERR_INVALID_ARG      # < ceil(n/32)
    assert _pack(SD(2, 128, (1 << 26) + 1, 1 << 22)) == fa.FATHOM_ERR_UNSUPPORTED
    assert _pack(good, keys=None) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(good, keys=ctypes.c_void_p(0x1004)) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(good, stride_token=130) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(good, stride_head=100) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(good, planes=ctypes.c_void_p(0x1008)) == fa.FATHOM_ERR_INVALID_ARG
    assert _pack(good, ws=None) == fa.FATHOM_ERR_WORKSPACE
    assert _pack(good, ws_bytes=16) == fa.FATHOM_ERR_WORKSPACE
    assert _pack(good, ws=ctypes.c_void_p(0x1010)) == fa.FATHOM_ERR_WORKSPACE
    assert "workspace" in lib.fathom_last_error().decode()


def _alloc(store, num_q=8, group=4, budget=92, q=FAKE, alloc=FAKE):
    return lib.fathom_allocate(q, num_q, group, FAKE, ctypes.byref(store), budget, alloc, None)


def test_allocate_validation():
    s = SD(2, 128, 1000, 32)
    assert _alloc(s, num_q=6) == fa.FATHOM_ERR_INVALID_ARG                 # != H * group
    assert _alloc(s, budget=-1) == fa.FATHOM_ERR_INVALID_ARG
    assert _alloc(s, budget=513) == fa.FATHOM_ERR_INVALID_ARG
    assert _alloc(s, group=0) == fa.FATHOM_ERR_INVALID_ARG
    assert _alloc(s, q=None) == fa.FATHOM_ERR_INVALID_ARG
    assert _alloc(s, alloc=ctypes.c_void_p(0x1001)) == fa.FATHOM_ERR_INVALID_ARG
    assert _alloc(SD(2, 256, 1000, 32)) == fa.FATHOM_ERR_UNSUPPORTED
    assert "513" in (_alloc(s, budget=513) and lib.fathom_last_error().decode())


def _control(num_q=8, mode=0, budget=136, q=FAKE, alloc=FAKE):
    return lib.fathom_control_allocate(q, num_q, mode, budget, alloc, None)


def test_control_allocate_validation():
    assert _control(mode=2) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(mode=-1) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(budget=-1) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(budget=513) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(num_q=0) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(q=None) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(q=ctypes.c_void_p(0x1004)) == fa.FATHOM_ERR_INVALID_ARG
    assert _control(alloc=ctypes.c_void_p(0x1001)) == fa.FATHOM_ERR_INVALID_ARG
    assert "mode" in (_control(mode=5) and lib.fathom_last_error().decode())


def _scan(store, num_q=8, group=4, k=16, planes=FAKE, ws=FAKE, ws_bytes=1 << 30, out_idx=FAKE):
    return lib.fathom_scan_topk(planes, FAKE, FAKE, ctypes.byref(store), FAKE, FAKE, num_q, group, k,
                                out_idx, FAKE, None, ws, ws_bytes, None)


def test_scan_validation():
    s = SD(2, 128, 1000, 32)
    assert _scan(s, k=0) == fa.FATHOM_ERR_INVALID_ARG
    assert _scan(s, k=1001) == fa.FATHOM_ERR_INVALID_ARG
    big = SD(1, 128, 10000, fa.plane_ldw(10000))
    assert _scan(big, num_q=4, k=4097) == fa.FATHOM_ERR_UNSUPPORTED
    assert _scan(s, num_q=7) == fa.FATHOM_ERR_INVALID_ARG
    assert _scan(s, planes=ctypes.c_void_p(0x1004)) == fa.FATHOM_ERR_INVALID_ARG
    assert _scan(s, out_idx=None) == fa.FATHOM_ERR_INVALID_ARG
    assert _scan(s, ws_bytes=1024) == fa.FATHOM_ERR_WORKSPACE
    assert _scan(s, ws=None) == fa.FATHOM_ERR_WORKSPACE
    assert _scan(SD(2, 128, 1000, 36), ws_bytes=10) == fa.FATHOM_ERR_WORKSPACE


def _attend(store=None, num_q=8, group=4, k=16, scale=0.088, stride_token=128, krows=FAKE, ws=FAKE,
            ws_bytes=1 << 30):
    store = store or SD(2, 128, 1000, 32)
    return lib.fathom_sparse_attention(krows, FAKE, store.n * stride_token, stride_token, ctypes.byref(store),
                                       FAKE, FAKE, num_q, group, k, ctypes.c_float(scale), FAKE, ws, ws_bytes, None)


def test_attention_validation():
    assert _attend(num_q=7) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(k=0) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(k=1001) == fa.FATHOM_ERR_INVALID_ARG
    big = SD(1, 128, 10000, fa.plane_ldw(10000))
    assert _attend(store=big, num_q=4, k=4097) == fa.FATHOM_ERR_UNSUPPORTED
    assert _attend(scale=float("inf")) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(stride_token=132) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(stride_token=64) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(krows=ctypes.c_void_p(0x1008)) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(krows=None) == fa.FATHOM_ERR_INVALID_ARG
    assert _attend(ws_bytes=16) == fa.FATHOM_ERR_WORKSPACE
    assert _attend(store=SD(2, 256, 1000, 32)) == fa.FATHOM_ERR_UNSUPPORTED
    assert fa.workspace_bytes(fa.FATHOM_OP_ATTEND, SD(8, 128, 1 << 20, 32768), 32, 2048) == 32 * 16 * 130 * 4


def _append(store=None, m=1, stride_token=128, keys=FAKE, planes=FAKE):
    store = store or SD(2, 128, 1000, 32)
    return lib.fathom_append_keys(keys, m * stride_token, stride_token, m, ctypes.byref(store), planes, FAKE, FAKE,
                                  None)


def test_append_validation():
    assert _append(m=0) == fa.FATHOM_ERR_INVALID_ARG
    assert _append(m=25) == fa.FATHOM_ERR_INVALID_ARG          # 1000 + 25 > 32 * 32 words
    assert _append(stride_token=64) == fa.FATHOM_ERR_INVALID_ARG
    assert _append(keys=None) == fa.FATHOM_ERR_INVALID_ARG
    assert _append(planes=ctypes.c_void_p(0x1004)) == fa.FATHOM_ERR_INVALID_ARG
    assert _append(store=SD(2, 256, 1000, 32)) == fa.FATHOM_ERR_UNSUPPORTED
    assert "capacity" in (_append(m=25) and lib.fathom_last_error().decode())


def test_misc_validation():
    assert lib.fathom_host_device_pointer(None, None) == fa.FATHOM_ERR_INVALID_ARG
    assert lib.fathom_timing_read(None, None) == fa.FATHOM_ERR_INVALID_ARG


def test_per_head_block_limit():
    """The scan addresses one head's plane block with 32-bit byte offsets: a
    block of 2^32 bytes or more is rejected on the host (a larger legal ldw
    would otherwise wrap row offsets onto low rows)."""
    top = (1 << 21) - 4                       # largest ldw whose block is < 4 GiB
    ok = SD(1, 128, top * 32, top)
    assert fa.workspace_bytes(fa.FATHOM_OP_PACK, ok) > 0
    for n, ldw in (((1 << 26), 1 << 21), (1000, 1 << 21), (1000, 1 << 22)):
        s = SD(1, 128, n, ldw)
        assert fa.workspace_bytes(fa.FATHOM_OP_PACK, s) == 0
        assert _pack(s) == fa.FATHOM_ERR_UNSUPPORTED
        assert "addressable" in lib.fathom_last_error().decode()
        assert _scan(s, num_q=4, k=16) == fa.FATHOM_ERR_UNSUPPORTED
    # the whole store: 1025 heads of just under 4 GiB exceed 4 TiB
    assert _pack(SD(1025, 128, top * 32, top)) == fa.FATHOM_ERR_UNSUPPORTED


def test_stream_read_validation():
    assert lib.fathom_stream_read_sink_words() > 0
    assert lib.fathom_stream_read(None, 1 << 20, FAKE, None) == fa.FATHOM_ERR_INVALID_ARG
    assert lib.fathom_stream_read(FAKE, 1000, FAKE, None) == fa.FATHOM_ERR_INVALID_ARG
    assert lib.fathom_stream_read(ctypes.c_void_p(0x1008), 1 << 20, FAKE, None) == fa.FATHOM_ERR_INVALID_ARG


def test_noalloc_rejects_on_host():
    s = SD(65, 128, 1000, 32)
    st = lib.fathom_allocate_scan_topk_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.byref(s), FAKE, 65, 1, 92, 10, FAKE,
                                               FAKE, FAKE, None)
    assert st == fa.FATHOM_ERR_UNSUPPORTED and "allocation-free" in lib.fathom_last_error().decode()
    s = SD(2, 128, 1000, 32)
    assert lib.fathom_allocate_scan_topk_noalloc(FAKE, FAKE, FAKE, None, ctypes.byref(s), FAKE, 8, 4, 92, 10, FAKE,
                                                 FAKE, FAKE, None) == fa.FATHOM_ERR_INVALID_ARG


def test_staged_validation():
    s = SD(2, 128, 1000, 32)

    def call(num_q=8, group=4, budget=92, k=10, staging=FAKE, staging_bytes=1 << 30, ws_bytes=1 << 30, var=FAKE,
             mode=0):
        return lib.fathom_allocate_scan_topk_staged(FAKE, FAKE, FAKE, var, ctypes.byref(s), FAKE, num_q, group, budget,
                                                    k, FAKE, FAKE, FAKE, staging, staging_bytes, FAKE, ws_bytes, mode,
                                                    None, None)
    assert call(num_q=6) == fa.FATHOM_ERR_INVALID_ARG
    assert call(budget=600) == fa.FATHOM_ERR_INVALID_ARG
    assert call(k=0) == fa.FATHOM_ERR_INVALID_ARG
    assert call(var=None) == fa.FATHOM_ERR_INVALID_ARG
    assert call(staging=ctypes.c_void_p(0x1010)) == fa.FATHOM_ERR_INVALID_ARG
    assert call(staging_bytes=2 * 128 * 4 * 32 * 4 - 1) == fa.FATHOM_ERR_WORKSPACE
    assert call(ws_bytes=100) == fa.FATHOM_ERR_WORKSPACE
    assert call(mode=2) == fa.FATHOM_ERR_INVALID_ARG
    assert fa.staging_bytes(s) == 2 * 128 * 4 * 32 * 4
