"""Benchmark of the Fathom decode-step hot path on one MI355X.

One step = per-query allocation + plane-prefix scan with fused top-k over
every KV head of the workload, in one call (fathom_allocate_scan_topk), inputs
resident in HBM.  The default workload is the 1M-token Qwen3-8B-shaped decode
step: 8 KV heads x 1,048,576 keys x 128 channels, 32 query heads (GQA 4),
budget B = 92 bits, k = 2048.  Synthetic seeded keys (no model weights are
available).  Several copies of the plane store are rotated so that
consecutive steps never find their planes in the 256 MB Infinity Cache.

After the timed region, attention over the rows the step selected (bf16 K
and V, split over chunks of the selected rows, then combined) is timed too
("attention").

The same scan is also timed on the fixed-width reads the pages compare with
(136 and 68 bits per key: uniform depth, or whole 4-bit channels by |q|), as
control allocation + scan per step, beside the Fathom step made of the same
two calls ("controls").

Further sub-records, all after the timed region and never the headline:
the many-session shape ("multi_session"), a step in which one query takes
the exact fallback ("fallback"), the store in pinned host memory read over
PCIe ("host_resident"), and two ceilings measured in the same run
("ceilings": a hand-written streaming read of device memory, and a pinned
host-to-device copy).

Prints one JSON line (see the repository's design notes for the fields).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gkeys/s and achieved HBM GB/s (% peak) for scan+top-k, 1M keys, B=92 bits"
HBM_PEAK_GBS = 8000.0
TIMING_EVERY = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_main_qwen3_8b_1m_traffic.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def union_bytes(alloc: np.ndarray, group: int, ldw: int) -> int:
    """Plane bytes a step must read: per KV head, per channel, the longest
    prefix any of its queries reads (the union), times the row length."""
    Q, d = alloc.shape
    u = alloc.reshape(Q // group, group, d).max(axis=1).astype(np.int64)
    return int(u.sum()) * ldw * 4


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget, target_s):
    """Time the oracle (allocate + code-form scores + full-sort top-k) on one
    KV head's GQA group over a bounded key sample, single-threaded."""
    import threadpoolctl
    import oracle as O
    from sparse_kv_cache_amd import synth

    rng = np.random.default_rng(w.seed)
    keys = synth.head_keys(rng, w.n, w.d)
    _, lo, step, var, codes = O.pack_head(keys)
    del keys
    # the queries of head 0 (same draws the GPU run uses come after all
    # heads; the baseline only needs queries of the right distribution)
    q = np.random.default_rng(w.seed + 1000).standard_normal((w.group, w.d)).astype(np.float32)
    n_s = min(w.n, 1 << 16)
    done_keys, elapsed = 0, 0.0
    with threadpoolctl.threadpool_limits(1):
        while elapsed < target_s:
            start = (done_keys % w.n)
            sl = slice(start, min(start + n_s, w.n))
            t0 = time.perf_counter()
            for g in range(w.group):
                b = O.allocate(q[g], var, budget)
                s = O.scores_from_codes(codes[sl], lo, step, q[g], b)
                O.topk(s, min(w.k, s.shape[0]))
            elapsed += time.perf_counter() - t0
            done_keys += sl.stop - sl.start
    return {
        "value": done_keys / elapsed / 1e9,
        "unit": "Gkeys/s",
        "cores": 1,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"KV head 0 of the workload, {done_keys} keys scored for its {w.group} query heads "
                  f"(allocate + float64 code-form scores + full-sort top-k, k={w.k}) in slices of "
                  f"{n_s} keys, {elapsed:.1f} s, NumPy single thread",
    }


def device_keys(w, dev, torch):
    """Keys of workload w drawn on the device with the same recipe as
    sparse_kv_cache_amd.synth (per head: log-normal channel scales, four
    outlier channels x 8, Gaussian keys), from a torch generator: the same
    distribution, not the same bytes.  Used only for timing sub-records."""
    from sparse_kv_cache_amd import synth
    rng = np.random.default_rng(w.seed)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    keys = torch.empty((w.num_kv_heads, w.n, w.d), dtype=torch.float32, device=dev)
    for h in range(w.num_kv_heads):
        sigma = rng.lognormal(0.0, 0.5, w.d).astype(np.float32)
        sigma[rng.choice(w.d, synth.OUTLIER_CHANNELS, replace=False)] *= synth.OUTLIER_SCALE
        torch.randn((w.n, w.d), generator=gen, device=dev, out=keys[h])
        keys[h].mul_(torch.from_numpy(sigma).to(dev)[None, :])
    q = rng.standard_normal((w.num_q, w.d)).astype(np.float32)
    return keys, q


def timed_loop(fn, steps, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def kernel_timed_loop(fn, steps, fa, torch):
    """Wall time per call, and the main scan kernel's mean duration from the
    events its own dispatch carries (every TIMING_EVERY-th call)."""
    fa.timing_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        timed = i % TIMING_EVERY == 0
        if timed:
            fa.timing_enable(True)
        fn(i)
        if timed:
            fa.timing_enable(False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    tot, launches = fa.timing_read()
    return ms, (tot / launches if launches else float("nan"))


def stream_ceiling(dev, fa, torch, gib=2, reps=10):
    """GB/s of a plain hand-written streaming read of `gib` GiB of device
    memory (far above the 256 MB Infinity Cache), timed with events on the
    stream the kernel runs on."""
    buf = torch.zeros(gib * (1 << 28), dtype=torch.int32, device=dev)
    sink = torch.zeros(int(fa.lib.fathom_stream_read_sink_words()), dtype=torch.int32, device=dev)
    for _ in range(2):
        fa.stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fa.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    return {"gbs": round(gib * (1 << 30) / (ms * 1e-3) / 1e9, 1), "bytes": gib * (1 << 30), "ms": round(ms, 4),
            "kernel": "stream_read_kernel (16-byte non-temporal loads, 2048 workgroups)"}


def pcie_ceiling(dev, torch, mib=512, reps=5):
    """GB/s of a pinned host-to-device copy (the copy engines over PCIe)."""
    src = torch.empty(mib * (1 << 18), dtype=torch.int32, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(src.shape, dtype=torch.int32, device=dev)
    dst.copy_(src, non_blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"gbs": round(mib * (1 << 20) / (ms * 1e-3) / 1e9, 1), "bytes": mib * (1 << 20), "ms": round(ms, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_8b_1m")
    ap.add_argument("--budget", type=int, default=None)
    ap.add_argument("--copies", type=int, default=3, help="plane-store copies rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="leave the main-kernel timing events off (for traces of the bare step)")
    ap.add_argument("--control-steps", type=int, default=50,
                    help="steps per fixed-width control read (0: skip the controls)")
    ap.add_argument("--host-steps", type=int, default=10,
                    help="steps with the plane store in pinned host memory, read over PCIe (0: skip)")
    ap.add_argument("--attention-steps", type=int, default=50,
                    help="steps of attention over the selected rows (0: skip)")
    ap.add_argument("--multi-steps", type=int, default=50,
                    help="steps of the many-session shape at each of its budgets (0: skip)")
    ap.add_argument("--fallback-steps", type=int, default=10,
                    help="steps with one all-zero query, which takes the exact fallback (0: skip)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the streaming-read and PCIe ceilings")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the plane store shards by KV head or session with no exchange; see the design notes)",
              file=sys.stderr)
        return 2

    import torch
    from sparse_kv_cache_amd import fathom as fa
    from sparse_kv_cache_amd import synth
    from sparse_kv_cache_amd.profiling import source_digest

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    budget = args.budget if args.budget is not None else w.budgets[0]
    H, n, d, G, Q, k = w.num_kv_heads, w.n, w.d, w.group, w.num_q, w.k
    store = fa.store_desc(H, n, d)
    log(f"workload {w.name}: H={H} n={n} d={d} Q={Q} G={G} B={budget} k={k}")

    # ---- inputs: keys -> device -> packed planes (pack timed once, for the record)
    t0 = time.perf_counter()
    keys = torch.empty((H, n, d), dtype=torch.float32, device=dev)
    q_np = None
    for kind, *rest in synth.stream_inputs(w.seed, H, n, Q, d):
        if kind == "head":
            h, kh = rest
            keys[h].copy_(torch.from_numpy(kh))
        else:
            q_np = rest[0]
    torch.cuda.synchronize()
    log(f"generated keys in {time.perf_counter() - t0:.1f} s")
    planes0 = torch.empty((H, d, 4, store.ldw), dtype=torch.int32, device=dev)
    pack_ws = fa.alloc_workspace(fa.workspace_bytes(fa.FATHOM_OP_PACK, store), dev)
    fa.pack_planes(keys, store, planes=planes0, workspace=pack_ws)   # warm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _, lo, step, var = fa.pack_planes(keys, store, planes=planes0, workspace=pack_ws)
    e1.record()
    torch.cuda.synchronize()
    pack_ms = e0.elapsed_time(e1)
    # bf16 K and V rows for the attention over the selected keys (V drawn on
    # the device from a fixed seed)
    k_bf16 = keys.to(torch.bfloat16) if args.attention_steps > 0 else None
    del keys
    torch.cuda.empty_cache()
    copies = [planes0] + [planes0.clone() for _ in range(max(1, args.copies) - 1)]
    qd = torch.from_numpy(q_np).to(dev)
    alloc = torch.empty((Q, d), dtype=torch.uint8, device=dev)
    out_idx = torch.empty((Q, k), dtype=torch.int32, device=dev)
    out_score = torch.empty((Q, k), dtype=torch.float32, device=dev)
    scan_ws = fa.alloc_workspace(fa.workspace_bytes(fa.FATHOM_OP_SCAN, store, Q, k), dev)

    def step_fn(i):
        # allocation and scan + top-k in one call (the allocation is computed
        # inside the scan's first kernel)
        fa.allocate_scan_topk(copies[i % len(copies)], lo, step, var, store, qd, G, budget, k,
                              workspace=scan_ws, alloc=alloc, out_idx=out_idx, out_score=out_score)

    if not args.no_kernel_timing:
        fa.timing_enable(True)    # creates the event pool outside the timed region
    for i in range(args.warmup):
        step_fn(i)
    fa.timing_enable(False)
    torch.cuda.synchronize()
    alg_plane_bytes = union_bytes(alloc.cpu().numpy(), G, store.ldw)
    alg_bytes = alg_plane_bytes + H * d * 8 + Q * d * 5 + Q * k * 8

    if args.calibrate_copy_mib:
        nel = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # one elementwise kernel: reads and writes nel*4 bytes
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy_mib} MiB read + written per launch, 3 launches")
        del src, dst

    # ---- the timed region.  The main kernel's duration is read from HIP
    # events carried by its own dispatch, on every TIMING_EVERY-th step
    # (events on every launch would add their own gaps to the step).
    fa.timing_read()   # clear the record
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        timed = not args.no_kernel_timing and i % TIMING_EVERY == 0
        if timed:
            fa.timing_enable(True)
        step_fn(i)
        if timed:
            fa.timing_enable(False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    main_ms_total, launches = fa.timing_read()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    main_ms = main_ms_total / launches if launches else float("nan")
    gkeys = H * n / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (main_ms * 1e-3) / 1e9
    step_achieved = alg_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- ceilings measured in the same run
    ceilings = None
    if not args.no_ceilings:
        ceilings = {"hbm_stream_read": stream_ceiling(dev, fa, torch), "pcie_h2d_copy": pcie_ceiling(dev, torch)}
        log(f"ceilings: stream read {ceilings['hbm_stream_read']['gbs']} GB/s, "
            f"pinned H2D copy {ceilings['pcie_h2d_copy']['gbs']} GB/s")

    # ---- fixed-width control reads through the same scan, each as control
    # allocation + scan, beside the Fathom step made of the same two calls
    controls = {}
    if args.control_steps > 0:
        def two_call_step(i):
            fa.allocate(qd, var, G, budget, store, out=alloc)
            fa.scan_topk(copies[i % len(copies)], lo, step, store, qd, alloc, G, k,
                         workspace=scan_ws, out_idx=out_idx, out_score=out_score)
        for i in range(5):
            two_call_step(i)
        f2_ms = timed_loop(two_call_step, args.control_steps, torch)
        controls["fathom_two_calls"] = {"ms_per_step": round(f2_ms, 4), "budget_bits": budget,
                                        "union_bits_per_key": round(alg_plane_bytes * 8 / (H * store.ldw * 32), 2)}
        ctrl_alloc = torch.empty((Q, d), dtype=torch.uint8, device=dev)
        for name, mode, width in (("top_channels_136", fa.FATHOM_CONTROL_TOP_CHANNELS, 136),
                                  ("uniform_136", fa.FATHOM_CONTROL_UNIFORM, 136),
                                  ("top_channels_68", fa.FATHOM_CONTROL_TOP_CHANNELS, 68)):
            def ctrl_step(i):
                fa.control_allocate(qd, mode, width, out=ctrl_alloc)
                fa.scan_topk(copies[i % len(copies)], lo, step, store, qd, ctrl_alloc, G, k,
                             workspace=scan_ws, out_idx=out_idx, out_score=out_score)
            for i in range(5):
                ctrl_step(i)
            c_ms = timed_loop(ctrl_step, args.control_steps, torch)
            c_bytes = union_bytes(ctrl_alloc.cpu().numpy(), G, store.ldw)
            controls[name] = {
                "ms_per_step": round(c_ms, 4),
                "gkeys_per_s": round(H * n / (c_ms * 1e-3) / 1e9, 3),
                "union_bits_per_key": round(c_bytes * 8 / (H * store.ldw * 32), 2),
                "fathom_speedup": round(c_ms / f2_ms, 3),
            }
            log(f"control {name}: {c_ms * 1e3:.1f} us/step")

    # ---- one query of the step is all zero: every score ties, the candidate
    # list overflows and that query takes the exact fallback
    fallback = None
    if args.fallback_steps > 0:
        q_fb = qd.clone()
        q_fb[0].zero_()
        f_alloc = torch.empty_like(alloc)

        def fb_step(i):
            fa.allocate_scan_topk(copies[i % len(copies)], lo, step, var, store, q_fb, G, budget, k,
                                  workspace=scan_ws, alloc=f_alloc, out_idx=out_idx, out_score=out_score)
        fb_step(0)
        fb_ms = timed_loop(fb_step, args.fallback_steps, torch)
        fallback = {"ms_per_step": round(fb_ms, 4), "zero_queries": 1, "vs_step": round(fb_ms / ms_per_step, 2)}
        log(f"step with one zero query (exact fallback): {fb_ms * 1e3:.1f} us/step")

    # ---- the same step with the plane store in pinned host memory, read
    # zero-copy over PCIe (never the headline value)
    host_resident = None
    if args.host_steps > 0:
        pinned = torch.empty(planes0.shape, dtype=planes0.dtype, pin_memory=True)
        pinned.copy_(planes0)
        torch.cuda.synchronize()
        hptr = fa.host_device_pointer(pinned)
        h_alloc = torch.empty_like(alloc)
        host_resident = {}
        for hb in sorted(set(synth.WORKLOADS["host_resident"].budgets) | {budget}):
            def host_step(i):
                fa.allocate_scan_topk(planes0, lo, step, var, store, qd, G, hb, k, workspace=scan_ws, alloc=h_alloc,
                                      out_idx=out_idx, out_score=out_score, planes_ptr=hptr)
            host_step(0)
            h_ms = timed_loop(host_step, args.host_steps, torch)
            hb_bytes = union_bytes(h_alloc.cpu().numpy(), G, store.ldw)
            rec = {
                "ms_per_step": round(h_ms, 4),
                "gkeys_per_s": round(H * n / (h_ms * 1e-3) / 1e9, 3),
                "union_bytes": hb_bytes,
                "pcie_gbs": round(hb_bytes / (h_ms * 1e-3) / 1e9, 1),
            }
            if ceilings:
                rec["frac_of_pcie_copy"] = round(rec["pcie_gbs"] / ceilings["pcie_h2d_copy"]["gbs"], 3)
            host_resident[f"B{hb}_zero_copy"] = rec
            log(f"host-resident store, B={hb}, zero-copy: {h_ms * 1e3:.1f} us/step")
        # the union rows staged by the copy engines, head by head, overlapped
        # with the scans (the call waits for the allocation on the host)
        staging = fa.alloc_workspace(fa.staging_bytes(store), dev)
        st_ws = fa.alloc_workspace(fa.workspace_bytes(fa.FATHOM_OP_SCAN, store, G, k), dev)
        copy_stream = torch.cuda.Stream(device=dev)
        for mname, smode in (("gather", fa.FATHOM_STAGE_GATHER), ("copy_engine", fa.FATHOM_STAGE_COPY_ENGINE)):
            for hb in sorted(set(synth.WORKLOADS["host_resident"].budgets) | {budget}):
                def staged_step(i):
                    fa.allocate_scan_topk_staged(pinned, lo, step, var, store, qd, G, hb, k, staging=staging,
                                                 workspace=st_ws, alloc=h_alloc, out_idx=out_idx, out_score=out_score,
                                                 mode=smode, copy_stream=copy_stream)
                staged_step(0)
                s_ms = timed_loop(staged_step, args.host_steps, torch)
                hb_bytes = union_bytes(h_alloc.cpu().numpy(), G, store.ldw)
                rec = {
                    "ms_per_step": round(s_ms, 4),
                    "gkeys_per_s": round(H * n / (s_ms * 1e-3) / 1e9, 3),
                    "union_bytes": hb_bytes,
                    "pcie_gbs": round(hb_bytes / (s_ms * 1e-3) / 1e9, 1),
                    "vs_zero_copy": round(host_resident[f"B{hb}_zero_copy"]["ms_per_step"] / s_ms, 3),
                }
                if ceilings:
                    rec["frac_of_pcie_copy"] = round(rec["pcie_gbs"] / ceilings["pcie_h2d_copy"]["gbs"], 3)
                host_resident[f"B{hb}_staged_{mname}"] = rec
                log(f"host-resident store, B={hb}, staged ({mname}): {s_ms * 1e3:.1f} us/step")
        del pinned, staging, st_ws

    # ---- attention over the rows the last step selected
    attention = None
    if args.attention_steps > 0:
        fa.allocate_scan_topk(copies[0], lo, step, var, store, qd, G, budget, k, workspace=scan_ws, alloc=alloc,
                              out_idx=out_idx, out_score=out_score)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed + 7)
        v_bf16 = torch.randn((H, n, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        att_ws = fa.alloc_workspace(fa.workspace_bytes(fa.FATHOM_OP_ATTEND, store, Q, k), dev)
        att_out = torch.empty((Q, d), dtype=torch.float32, device=dev)
        for _ in range(5):
            fa.sparse_attention(k_bf16, v_bf16, store, qd, out_idx, G, out=att_out, workspace=att_ws)
        a_ms = timed_loop(lambda i: fa.sparse_attention(k_bf16, v_bf16, store, qd, out_idx, G, out=att_out,
                                                        workspace=att_ws), args.attention_steps, torch)
        a_bytes = Q * k * 2 * d * 2 + Q * k * 4 + Q * d * 8
        attention = {
            "ms_per_step": round(a_ms, 4),
            "rows_per_step": Q * k,
            "gbs": round(a_bytes / (a_ms * 1e-3) / 1e9, 1),
            "decode_step_ms": round(ms_per_step + a_ms, 4),
        }
        log(f"attention over the selected rows: {a_ms * 1e3:.1f} us/step")
        del v_bf16, k_bf16
    del copies[1:]
    torch.cuda.empty_cache()

    # ---- the many-session shape (128 KV heads = 16 sessions x 8, 131,072 keys,
    # 512 query heads, k = 1024), keys drawn on the device
    multi = None
    if args.multi_steps > 0 and w.name != "multi_session":
        mw = synth.WORKLOADS["multi_session"]
        mkeys, mq = device_keys(mw, dev, torch)
        mstore = fa.store_desc(mw.num_kv_heads, mw.n, mw.d)
        mplanes, mlo, mstep, mvar = fa.pack_planes(mkeys, mstore)
        del mkeys
        torch.cuda.empty_cache()
        mcopies = [mplanes, mplanes.clone()]
        mqd = torch.from_numpy(mq).to(dev)
        mQ = mw.num_q
        m_alloc = torch.empty((mQ, mw.d), dtype=torch.uint8, device=dev)
        m_idx = torch.empty((mQ, mw.k), dtype=torch.int32, device=dev)
        m_val = torch.empty((mQ, mw.k), dtype=torch.float32, device=dev)
        m_ws = fa.alloc_workspace(fa.workspace_bytes(fa.FATHOM_OP_SCAN, mstore, mQ, mw.k), dev)
        multi = {"kv_heads": mw.num_kv_heads, "keys_per_head": mw.n, "query_heads": mQ, "k": mw.k,
                 "keys": "drawn on the device (same recipe, torch generator)"}
        fa.timing_enable(True)
        fa.timing_enable(False)
        for mb in mw.budgets:
            def m_step(i):
                fa.allocate_scan_topk(mcopies[i % 2], mlo, mstep, mvar, mstore, mqd, mw.group, mb, mw.k,
                                      workspace=m_ws, alloc=m_alloc, out_idx=m_idx, out_score=m_val)
            for i in range(5):
                m_step(i)
            m_ms, m_main = kernel_timed_loop(m_step, args.multi_steps, fa, torch)
            mb_plane = union_bytes(m_alloc.cpu().numpy(), mw.group, mstore.ldw)
            mb_bytes = mb_plane + mw.num_kv_heads * mw.d * 8 + mQ * mw.d * 5 + mQ * mw.k * 8
            multi[f"B{mb}"] = {
                "ms_per_step": round(m_ms, 4),
                "gkeys_per_s": round(mw.num_kv_heads * mw.n / (m_ms * 1e-3) / 1e9, 3),
                "main_kernel_ms": round(m_main, 4),
                "alg_bytes_per_step": mb_bytes,
                "union_bits_per_key": round(mb_plane * 8 / (mw.num_kv_heads * mstore.ldw * 32), 2),
                "main_kernel_frac": round(mb_bytes / (m_main * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "step_frac": round(mb_bytes / (m_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            log(f"multi_session B={mb}: {m_ms * 1e3:.1f} us/step, main kernel {m_main * 1e3:.1f} us")
        del mcopies, mplanes
        torch.cuda.empty_cache()

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_digest") == source_digest() and tr.get("budget") == budget:
            traffic = tr.get("bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w, budget, args.cpu_seconds)

    roofline = {
        "bound": "hbm",
        "kernel": "scan_main_kernel",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "step_achieved": round(step_achieved, 1),
        "step_frac": round(step_achieved / HBM_PEAK_GBS, 4),
    }
    if ceilings:
        sc = ceilings["hbm_stream_read"]["gbs"]
        roofline["stream_ceiling"] = sc
        roofline["frac_of_stream_ceiling"] = round(achieved / sc, 4)
        roofline["step_frac_of_stream_ceiling"] = round(step_achieved / sc, 4)

    rec = {
        "metric": METRIC,
        "value": round(gkeys, 3),
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "score_arithmetic": "int8 matrix-core digits of 30-bit fixed-point plane weights, exact int32 sums, "
                            "fp32 scores",
        "data": "synthetic",
        "config": {
            "workload": w.name, "kv_heads": H, "keys_per_head": n, "d": d, "query_heads": Q,
            "gqa_group": G, "budget_bits": budget, "k": k, "store_copies": max(1, args.copies),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gscores_per_s": round(Q * n / (ms_per_step * 1e-3) / 1e9, 3),
        "alg_bytes_per_step": alg_bytes,
        "union_bits_per_key": round(alg_plane_bytes * 8 / (H * store.ldw * 32), 2),
        "main_kernel_ms": round(main_ms, 4),
        "step_gbs": round(step_achieved, 1),
        "pack_ms": round(pack_ms, 3),
        "ceilings": ceilings,
        "controls": controls,
        "fallback": fallback,
        "attention": attention,
        "host_resident": host_resident,
        "multi_session": multi,
        "kernel_source": source_digest(),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
