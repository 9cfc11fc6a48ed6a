"""Throughput of the rotated Top-K sparse SwiGLU MLP (LLaMA2-7B shape) at batch 1.

One step = one decode token through the whole path: rotate the 4096-wide
input (dense 4096² rotation), select its top 2457 channels, gather-product
the kept rows of the folded gate|up weight (4096→22016), SiLU(gate)·up,
rotate the 11008-wide result (4×2752 block rotation), select 6604 channels,
gather-product the kept rows of the folded down weight (11008→4096). Inputs
are seeded synthetic tensors of that shape; the weights are random-init.

Prints one JSON line. Timing: W untimed warm-up steps, then K steps between
two HIP events on the library's stream, with torch.cuda.synchronize() on
both sides. The weights are held in several copies that the steps cycle
through, so the 256 MB on-package cache cannot serve a repeated step.

Also reported: the dominant kernel (the gate|up gather product) timed on its
own with HIP events, against the HBM roofline; the dense product over the
same folded weight (this library's dense kernel and torch.matmul); and the
CPU oracle timed on the host on a bounded sample of tokens.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
COPY_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gather_vec_kernel": ["gather.hip", "common.hpp"],
    "select_gather_kernel": ["select_gather.hip", "select_core.hpp", "common.hpp"],
    "fused_linear_kernel": ["fused.hip", "select_core.hpp", "common.hpp"],
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "rotated_top_activation_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=0, help="weight copies (0: enough for 1 GiB)")
    p.add_argument("--mode", choices=["unfused", "fused", "best"], default="best")
    p.add_argument("--sparsity", type=int, default=40)
    p.add_argument("--q2-block", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-only", choices=["", "gather", "topk1", "fused1", "step", "copy"],
                   default="",
                   help="only launch that work (for profiler runs)")
    return p.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rotated_top_activation_amd import _lib, workloads as wl
    from rotated_top_activation_amd.device import RotatedLinear

    _lib.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if a.kernel_only == "copy":
        # A plain device copy of a known size (512 MiB read + 512 MiB written
        # per launch): the calibration for the HBM traffic counters.
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        return
    case = wl.llama7b_mlp(batch=1, sparsity_pct=a.sparsity, q2_block=a.q2_block or None)
    t0 = time.time()
    x, q1, wgu, q2, wd = wl.mlp_case_inputs(case)
    gen_s = time.time() - t0
    l1 = RotatedLinear(q1, wgu, "bf16", case.k1, keep_w=False)
    l2 = RotatedLinear(q2, wd, "bf16", case.k2, keep_w=False)
    torch.cuda.synchronize()

    # Enough copies that about 2.5 GiB of other weights pass between two uses
    # of one copy: the 256 MB on-package cache then serves almost none of a
    # step's reads.
    per_copy = sum(t.numel() * t.element_size() for t in (l1.Qt, l1.Wf, l2.Qt, l2.Wf))
    copies = a.copies or max(2, math.ceil((5 << 29) / per_copy) + 1)
    qt1 = [l1.Qt] + [l1.Qt.clone() for _ in range(copies - 1)]
    wf1 = [l1.Wf] + [l1.Wf.clone() for _ in range(copies - 1)]
    # gate|up folded weight with gate and up columns interleaved, so the
    # product writes SiLU(gate)·up directly
    wil1 = []
    for c in range(copies):
        t = torch.empty_like(l1.Wf)
        _lib.larosa_interleave_gate_up(wf1[c], t, case.d, case.f)
        wil1.append(t)
    qt2 = [l2.Qt] + [l2.Qt.clone() for _ in range(copies - 1)]
    wf2 = [l2.Wf] + [l2.Wf.clone() for _ in range(copies - 1)]

    d, f = case.d, case.f
    x_d = wl.to_torch(x, "bf16")
    gu = torch.empty((1, 2 * f), dtype=torch.bfloat16, device=dev)
    h = torch.empty((1, f), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, d), dtype=torch.bfloat16, device=dev)
    ws1 = l1.workspace(1, _lib.FUSED)
    ws2 = l2.workspace(1, _lib.FUSED)
    ws1s = torch.zeros(_lib.larosa_swiglu_workspace_bytes(1, d, f, case.k1, _lib.FUSED),
                       dtype=torch.uint8, device=dev)

    def step(i, mode):
        c = i % copies
        _lib.larosa_swiglu_layer_forward(x_d, qt1[c], l1.q_block, wil1[c], 1, d, f, case.k1, h,
                                         mode=mode, ws=ws1s)
        _lib.larosa_layer_forward(h, qt2[c], l2.q_block, wf2[c], 1, f, d, case.k2, y,
                                  mode=mode, ws=ws2)

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    modes = {"unfused": _lib.UNFUSED, "fused": _lib.FUSED}

    def capture(mode):
        # One HIP graph per weight copy: a replay launches the whole step.
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0, mode)  # warm the path on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c, mode)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    if a.kernel_only == "step":
        gs = capture(_lib.UNFUSED if a.mode != "fused" else _lib.FUSED)
        for i in range(a.steps):
            gs[i % copies].replay()
        torch.cuda.synchronize()
        return
    step_ms = {}
    eager_ms = {}
    graph_ms = {}
    if a.kernel_only == "":
        for name in (["unfused", "fused"] if a.mode == "best" else [a.mode]):
            eager_ms[name] = timed(lambda i, m=modes[name]: step(i, m), a.steps, a.warmup)
            gs = capture(modes[name])
            graph_ms[name] = timed(lambda i, g=gs: g[i % copies].replay(), a.steps, a.warmup)
            step_ms[name] = min(eager_ms[name], graph_ms[name])

    # The dominant kernels alone, gate|up (the larger linear): the one-token
    # selection folded into the product (unfused mode), the fused
    # rotate-select-gather, and for reference the product over a given row list.
    xr1 = torch.empty((1, d), dtype=torch.float32, device=dev)
    idx1 = torch.empty((1, case.k1), dtype=torch.int32, device=dev)
    val1 = torch.empty((1, case.k1), dtype=torch.float32, device=dev)
    _lib.larosa_rotate(x_d, l1.Qt, l1.q_block, xr1, 1, d)
    _lib.larosa_topk_select(xr1, 1, d, case.k1, idx1, val1)
    xr2 = torch.empty((1, f), dtype=torch.float32, device=dev)
    step(0, _lib.UNFUSED)  # h of this input
    _lib.larosa_rotate(h, l2.Qt, l2.q_block, xr2, 1, f)
    torch.cuda.synchronize()

    def topk1(i):
        _lib.larosa_topk_gemv(xr1, d, case.k1, wf1[i % copies], gu, 2 * f, ws=ws1)

    def topk2(i):
        _lib.larosa_topk_gemv(xr2, f, case.k2, wf2[i % copies], y, d, ws=ws2)

    def gather(i):
        _lib.larosa_sparse_gemv(idx1, None, case.k1, val1, wf1[i % copies], gu, 1, d, 2 * f,
                                ws=ws1)

    def fused1(i):
        c = i % copies
        _lib.larosa_layer_forward(x_d, qt1[c], l1.q_block, wf1[c], 1, d, 2 * f, case.k1, gu,
                                  mode=_lib.FUSED, ws=ws1)
    if a.kernel_only in ("gather", "topk1", "fused1"):
        fn = {"gather": gather, "topk1": topk1, "fused1": fused1}[a.kernel_only]
        for i in range(a.steps):
            fn(i)
        torch.cuda.synchronize()
        return
    topk1_ms = timed(topk1, a.steps, a.warmup)
    topk1_bytes = case.k1 * 2 * f * 2 + d * 4 + 2 * f * 2
    gather_ms = timed(gather, a.steps, a.warmup)
    gather_bytes = case.k1 * 2 * f * 2 + case.k1 * 8 + 2 * f * 2
    fused1_ms = timed(fused1, a.steps, a.warmup)
    fused1_bytes = l1.Qt.numel() * 2 + d * 2 + case.k1 * 2 * f * 2 + 2 * f * 2

    # Dense product over all rows of the same folded weight.
    def dense(i):
        _lib.larosa_dense_gemv(x_d, wf1[i % copies], gu, 1, d, 2 * f, ws=ws1)
    dense_ms = timed(dense, a.steps, a.warmup)
    dense_bytes = d * 2 * f * 2
    out_t = torch.empty((1, 2 * f), dtype=torch.bfloat16, device=dev)

    def tmm(i):
        torch.matmul(x_d, wf1[i % copies], out=out_t)
    torch_ms = timed(tmm, a.steps, a.warmup)

    # Per-stage times of the unfused step (each stage alone, cycling copies).
    stage = {}
    stage["rotate1"] = timed(lambda i: _lib.larosa_rotate(x_d, qt1[i % copies], l1.q_block, xr1,
                                                          1, d), a.steps, a.warmup)
    stage["select_gather1"] = topk1_ms
    stage["swiglu_alone"] = timed(lambda i: _lib.larosa_swiglu(gu, h, 1, f), a.steps, a.warmup)
    stage["rotate2"] = timed(lambda i: _lib.larosa_rotate(h, qt2[i % copies], l2.q_block, xr2,
                                                          1, f), a.steps, a.warmup)
    stage["select_gather2"] = timed(topk2, a.steps, a.warmup)
    stage["select1_alone"] = timed(lambda i: _lib.larosa_topk_select(xr1, 1, d, case.k1, idx1,
                                                                     val1), a.steps, a.warmup)
    stage["gather1_alone"] = gather_ms

    q_bytes = (l1.Qt.numel() + l2.Qt.numel()) * 2
    sparse_bytes = q_bytes + (case.k1 * 2 * f + case.k2 * d) * 2
    dense_mlp_bytes = (d * 2 * f + f * d) * 2
    best = min(step_ms, key=step_ms.get)
    ms = step_ms[best]
    def gbs(nbytes, ms_):
        return nbytes / (ms_ * 1e-3) / 1e9
    kernels = {
        "select_gather_kernel": dict(achieved=gbs(topk1_bytes, topk1_ms), bytes=topk1_bytes,
                                     us=topk1_ms * 1e3,
                                     what="one-token selection folded into the product, gate|up"),
        "gather_vec_kernel": dict(achieved=gbs(gather_bytes, gather_ms), bytes=gather_bytes,
                                  us=gather_ms * 1e3,
                                  what="product over a given kept-row list, gate|up"),
        "fused_linear_kernel": dict(achieved=gbs(fused1_bytes, fused1_ms), bytes=fused1_bytes,
                                    us=fused1_ms * 1e3, what="fused rotate-select-gather, gate|up"),
    }
    dom = "fused_linear_kernel" if best == "fused" else "select_gather_kernel"
    kd = kernels[dom]

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(case, x, q1, wgu, q2, wd, a.cpu_seconds)

    out = {
        "metric": "tokens/s and achieved HBM GB/s (% peak) of rotated Top-K sparse GEMV, 7B MLP",
        "value": round(1.0 / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "LLaMA2-7B-shaped SwiGLU MLP decode, rotated Top-K sparse, batch 1",
            "d": d, "ffn": f, "batch": 1, "sparsity": a.sparsity / 100,
            "k_in": case.k1, "k_down": case.k2, "q1_block": case.q1_block,
            "q2_block": case.q2_block, "mode": best, "weight_copies": copies,
            "launch": "hip graph" if graph_ms.get(best, 1e9) <= eager_ms.get(best, 1e9) else "eager",
        },
        "roofline": {
            "bound": "hbm", "kernel": f"{dom} ({kd['what']})",
            "achieved": round(kd["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kd["achieved"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom),
            "bytes_per_launch": kd["bytes"], "avg_us": round(kd["us"], 3),
        },
        "cpu_baseline": cpu,
        "detail": {
            "step_ms": {k: round(v, 5) for k, v in step_ms.items()},
            "eager_step_ms": {k: round(v, 5) for k, v in eager_ms.items()},
            "graph_step_ms": {k: round(v, 5) for k, v in graph_ms.items()},
            "mlp_sparse_bytes": sparse_bytes,
            "mlp_dense_weight_bytes": dense_mlp_bytes,
            "mlp_achieved_GBs": round(sparse_bytes / (ms * 1e-3) / 1e9, 1),
            "stage_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
            "kernels": {k: {"achieved_GBs": round(v["achieved"], 1), "bytes_per_launch": v["bytes"],
                            "avg_us": round(v["us"], 3), "frac": round(v["achieved"] / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(k)} for k, v in kernels.items()},
            "gate_up_dense_us": {"larosa_dense_gemv": round(dense_ms * 1e3, 2),
                                 "torch.matmul": round(torch_ms * 1e3, 2)},
            "gate_up_dense_GBs": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1),
            "gate_up_speedup_vs_dense": round(min(dense_ms, torch_ms) / topk1_ms, 3),
            "gate_up_gather_only_speedup_vs_dense": round(min(dense_ms, torch_ms) / gather_ms, 3),
            "input_gen_s": round(gen_s, 1),
        },
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(case, x, q1, wgu, q2, wd, seconds):
    """The oracle's MLP, as it stands, on the host: fold once (untimed), then
    as many single-token steps as fit in about `seconds`."""
    import numpy as np
    from oracle import larosa_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    w1 = ref.fold(q1, wgu, "bf16")
    w2 = ref.fold(q2, wd, "bf16")
    n = 0
    t0 = time.perf_counter()
    while True:
        ref.mlp(x, q1, w1, q2, w2, case.k1, case.k2, case.f)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} single-token steps of the same MLP (same x and weights), "
                      f"{el:.1f} s; fold done once beforehand, untimed"}


if __name__ == "__main__":
    main()
