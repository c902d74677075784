"""The allocation-free fused call (static scratch memory in the library)
against the workspace call it varies: identical allocations, indices and
scores, on two calls in a row, the second with a smaller input."""

import ctypes
import sys

import numpy as np
import pytest

import oracle as O
from sparse_kv_cache_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_cache_amd import fathom as fa  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _case(seed, H, n, G, B, k):
    keys, q = synth.make_inputs(seed, H, n, H * G)
    planes, lo, step, var = fa.pack_planes(torch.from_numpy(keys).to(DEV))
    store = fa.store_desc(H, n, 128)
    qd = torch.from_numpy(q).to(DEV)
    Q = H * G
    ref = fa.allocate_scan_topk(planes, lo, step, var, store, qd, G, B, k)
    alloc = torch.full((Q, 128), 7, dtype=torch.uint8, device=DEV)
    idx = torch.full((Q, k), -5, dtype=torch.int32, device=DEV)
    val = torch.full((Q, k), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    # through the C ABI itself
    st = fa.lib.fathom_allocate_scan_topk_noalloc(
        ctypes.c_void_p(planes.data_ptr()), ctypes.c_void_p(lo.data_ptr()), ctypes.c_void_p(step.data_ptr()),
        ctypes.c_void_p(var.data_ptr()), ctypes.byref(store), ctypes.c_void_p(qd.data_ptr()), Q, G, B, k,
        ctypes.c_void_p(alloc.data_ptr()), ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(val.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == fa.FATHOM_OK, fa.lib.fathom_last_error().decode()
    torch.cuda.synchronize()
    for a, b in zip(ref, (alloc, idx, val)):
        assert torch.equal(a.cpu(), b.cpu())
    var_h = var.cpu().numpy()
    assert np.array_equal(alloc.cpu().numpy(), O.allocate_all(q, var_h, G, B))


def test_noalloc_matches_workspace_call_twice_then_smaller():
    say("noalloc large")
    _case(401, 8, 200000, 4, 92, 2048)        # 32 query heads, 4 MiB-class scratch use
    say("noalloc smaller")
    _case(402, 2, 30011, 3, 136, 300)         # fewer heads, ragged n, a 3-query chunk


def test_noalloc_rejects_too_many_queries():
    store = fa.store_desc(65, 1000, 128)
    fake = ctypes.c_void_p(0x1000)
    st = fa.lib.fathom_allocate_scan_topk_noalloc(fake, fake, fake, fake, ctypes.byref(store), fake, 65, 1, 92, 10,
                                                  fake, fake, fake, None)
    assert st == fa.FATHOM_ERR_UNSUPPORTED
    assert "allocation-free" in fa.lib.fathom_last_error().decode()
